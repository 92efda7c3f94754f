"""Device-side synthetic stacks: draws SMOE-Q4 / SMOE-Q2 vaults in HBM with
libsmoe_synth.so (the device twin of synth.gen's code and scale streams) and
uploads host-drawn router weights, biases and hidden states."""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from . import gen

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsmoe_synth.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: python synth/build.py")
        L = ctypes.CDLL(LIB_PATH)
        L.synth_fill_experts.restype = ctypes.c_int
        L.synth_fill_experts.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.c_size_t, ctypes.c_void_p]
        L.synth_stream_read.restype = ctypes.c_int
        L.synth_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        _lib = L
    return _lib


def fill_experts(seed, dims, layer, e_begin, n_exp, dst_ptr, stride, stream=None):
    s = torch.cuda.current_stream().cuda_stream if stream is None else stream.cuda_stream
    rc = lib().synth_fill_experts(int(seed), dims.d_model, dims.d_ff, dims.chunk, dims.bits, int(layer), int(e_begin),
                                  int(n_exp), int(dst_ptr), int(stride), s)
    if rc != 0:
        raise RuntimeError(f"synth_fill_experts failed: {rc}")


def stream_read(buf: torch.Tensor, nbytes: int, offset: int = 0, grid: int = 0, sink=None, stream=None,
                start=None, stop=None):
    """One launch of the plain streaming-read reference over ``nbytes`` of the
    device tensor ``buf`` from byte ``offset``; ``start``/``stop`` are raw HIP
    events bracketing the launch (or None)."""
    if offset < 0 or offset % 16 or nbytes % 16 or offset + nbytes > buf.numel() * buf.element_size():
        raise ValueError("stream_read: range outside the buffer or not 16-byte aligned")
    if sink is None:
        sink = torch.empty(1024, dtype=torch.int32, device=buf.device)
    s = torch.cuda.current_stream().cuda_stream if stream is None else stream.cuda_stream
    rc = lib().synth_stream_read(buf.data_ptr() + offset, nbytes, int(grid), sink.data_ptr(), s, start, stop)
    if rc != 0:
        raise RuntimeError(f"synth_stream_read failed: {rc}")


def router_stack(seed, dims, n_layers, threads=8) -> np.ndarray:
    """Router gate weights of n_layers layers as bf16 bits [L][E][d] (uint16)."""
    with ThreadPoolExecutor(max_workers=threads) as ex:
        mats = list(ex.map(lambda L: gen.router_bits(seed, dims, L), range(n_layers)))
    return np.stack(mats)


def u16_to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


class DeviceStack:
    """A synthetic stack resident in HBM: vault [L][E] blobs, per-layer expert
    tables of blob pointers, router weights and optional Zipf logit biases."""

    def __init__(self, seed, dims, n_layers, zipf_s=0.0, device="cuda", experts=None):
        self.seed, self.dims, self.n_layers = seed, dims, n_layers
        E = dims.n_experts
        off = gen.blob_sections(dims)
        self.blob_bytes, self.stride = off["bytes"], off["stride"]
        self.vault = torch.empty(n_layers * E * self.stride, dtype=torch.uint8, device=device)
        base = self.vault.data_ptr()
        for L in range(n_layers):
            fill_experts(seed, dims, L, 0, E, base + L * E * self.stride, self.stride)
        ptrs = np.array([base + (L * E + e) * self.stride for L in range(n_layers) for e in range(E)],
                        dtype=np.int64)
        self.tables = torch.from_numpy(ptrs).to(device)
        self.router_bits = router_stack(seed, dims, n_layers)
        self.router = u16_to_device(self.router_bits, device)
        if zipf_s > 0:
            self.bias_np = np.stack([gen.zipf_bias(seed, dims, L, zipf_s) for L in range(n_layers)])
            self.bias = torch.from_numpy(self.bias_np).to(device)
        else:
            self.bias_np, self.bias = None, None

    def table(self, layer):
        E = self.dims.n_experts
        return self.tables[layer * E:(layer + 1) * E]

    def router_layer(self, layer):
        return self.router[layer]

    def bias_layer(self, layer):
        return None if self.bias is None else self.bias[layer]

    def blob(self, layer, expert) -> torch.Tensor:
        o = (layer * self.dims.n_experts + expert) * self.stride
        return self.vault[o:o + self.stride]
