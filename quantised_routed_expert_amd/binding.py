"""ctypes binding of libsmoe.so: argument marshalling only.

Every computation runs in the HIP library; this module turns torch tensors into
device pointers, the current torch stream into a hipStream_t, and status codes
into exceptions.  It fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsmoe.so")

SMOE_OK, SMOE_EINVAL, SMOE_EHIP, SMOE_ENOSLOT, SMOE_EBUSY, SMOE_ENOMEM = 0, -1, -2, -3, -4, -5

EXPORTED = [
    "smoe_last_error", "smoe_version", "smoe_blob_bytes", "smoe_blob_stride", "smoe_q4_blob_bytes",
    "smoe_q4_blob_stride",
    "smoe_workspace_bytes", "smoe_route", "smoe_moe_decode", "smoe_moe_decode_slots",
    "smoe_decode_layers", "smoe_moe_prefill_chunk", "smoe_ring_create", "smoe_ring_acquire",
    "smoe_ring_release", "smoe_ring_stats", "smoe_ring_log", "smoe_ring_destroy", "smoe_ring_acquire_table",
    "smoe_ring_prefetch", "smoe_ring_hottest", "smoe_route_ext", "smoe_ring_acquire_routed",
    "smoe_decode_layers_static",
]


class SmoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"smoe status {code}: {msg}")
        self.code = code


class SmoeDims(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("chunk", ctypes.c_int32), ("norm_topk_prob", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("quant_bits", ctypes.c_int32)]


class SmoeRingDesc(ctypes.Structure):
    _fields_ = [("n_slots", ctypes.c_int32), ("n_layers", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("slot_bytes", ctypes.c_size_t), ("slot_stride", ctypes.c_size_t),
                ("vault_layers", ctypes.POINTER(ctypes.c_void_p)), ("vault_stride", ctypes.c_size_t),
                ("slab_dev", ctypes.c_void_p), ("copy_stream", ctypes.c_void_p),
                ("log_capacity", ctypes.c_size_t)]


class SmoeRingEvent(ctypes.Structure):
    _fields_ = [("layer", ctypes.c_int32), ("rank", ctypes.c_int32), ("expert", ctypes.c_int32),
                ("kind", ctypes.c_int32), ("slot", ctypes.c_int32), ("evicted_layer", ctypes.c_int32),
                ("evicted_expert", ctypes.c_int32), ("pad", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded library; raises if it is missing (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() or "
                               f"python quantised_routed_expert_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        P, I, S, VP = ctypes.POINTER, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
        D = P(SmoeDims)
        sig = {
            "smoe_last_error": (ctypes.c_char_p, []),
            "smoe_version": (ctypes.c_int32, []),
            "smoe_blob_bytes": (S, [D]),
            "smoe_blob_stride": (S, [D]),
            "smoe_q4_blob_bytes": (S, [D]),
            "smoe_q4_blob_stride": (S, [D]),
            "smoe_workspace_bytes": (I, [D, ctypes.c_int32, P(S)]),
            "smoe_route": (I, [D, ctypes.c_int32, VP, VP, VP, VP, VP, VP, VP, S, VP]),
            "smoe_route_ext": (I, [D, ctypes.c_int32, VP, VP, VP, VP, VP, VP, ctypes.c_int32, VP, VP, S, VP]),
            "smoe_moe_decode": (I, [D, VP, VP, VP, VP, VP, VP, S, VP]),
            "smoe_moe_decode_slots": (I, [D, VP, VP, P(VP), VP, VP, S, VP]),
            "smoe_decode_layers": (I, [D, ctypes.c_int32, VP, VP, VP, VP, VP, VP, VP, P(VP), VP, S, VP]),
            "smoe_decode_layers_static": (I, [D, ctypes.c_int32, VP, VP, VP, VP, VP, VP, VP, VP]),
            "smoe_moe_prefill_chunk": (I, [D, ctypes.c_int32, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, S, P(VP), VP]),
            "smoe_ring_create": (I, [P(SmoeRingDesc), P(VP)]),
            "smoe_ring_acquire": (I, [VP, ctypes.c_int32, P(ctypes.c_int32), ctypes.c_int32, P(VP), VP]),
            "smoe_ring_release": (I, [VP]),
            "smoe_ring_acquire_table": (I, [VP, ctypes.c_int32, P(ctypes.c_int32), ctypes.c_int32, VP, VP]),
            "smoe_ring_acquire_routed": (I, [VP, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, VP, VP,
                                             P(ctypes.c_int32), P(ctypes.c_int32), VP]),
            "smoe_ring_prefetch": (I, [VP, ctypes.c_int32, P(ctypes.c_int32), ctypes.c_int32, P(ctypes.c_int32), VP]),
            "smoe_ring_hottest": (I, [VP, ctypes.c_int32, P(ctypes.c_int32), P(ctypes.c_int32), P(ctypes.c_uint64),
                                      P(ctypes.c_int32)]),
            "smoe_ring_stats": (I, [VP, P(ctypes.c_uint64), P(ctypes.c_uint64), P(ctypes.c_uint64),
                                    P(ctypes.c_uint64)]),
            "smoe_ring_log": (I, [VP, P(SmoeRingEvent), S, P(S)]),
            "smoe_ring_destroy": (I, [VP]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(code: int):
    if code != SMOE_OK:
        raise SmoeError(code, lib().smoe_last_error().decode())


def dims_struct(dims) -> SmoeDims:
    return SmoeDims(int(dims.d_model), int(dims.d_ff), int(dims.n_experts), int(dims.top_k), int(dims.chunk),
                    1 if dims.norm_topk_prob else 0, float(dims.rms_eps), int(getattr(dims, "bits", 4)))


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def blob_bytes(dims) -> int:
    return int(lib().smoe_blob_bytes(ctypes.byref(dims_struct(dims))))


def blob_stride(dims) -> int:
    return int(lib().smoe_blob_stride(ctypes.byref(dims_struct(dims))))


def workspace_bytes(dims, max_tokens: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().smoe_workspace_bytes(ctypes.byref(dims_struct(dims)), int(max_tokens), ctypes.byref(out)))
    return int(out.value)


def workspace(dims, max_tokens: int, device="cuda") -> torch.Tensor:
    """A zero-filled device workspace of the size the library asks for."""
    return torch.zeros(workspace_bytes(dims, max_tokens), dtype=torch.uint8, device=device)


def route(dims, residual, x_out, w_router, bias, topk_idx, topk_w, ws, stream=None):
    n_tok = residual.shape[0] if residual.dim() == 2 else 1
    _check(lib().smoe_route(ctypes.byref(dims_struct(dims)), int(n_tok), _ptr(residual), _ptr(x_out),
                            _ptr(w_router), _ptr(bias), _ptr(topk_idx), _ptr(topk_w), _ptr(ws),
                            ws.numel() if ws is not None else 0, _stream(stream)))


def route_ext(dims, residual, x_out, w_router, bias, topk_idx, topk_w, next_idx, ws, stream=None):
    """route(), plus next_idx [n_tok][n_next]: the experts at ranks k .. k + n_next - 1."""
    n_tok = residual.shape[0] if residual.dim() == 2 else 1
    n_next = next_idx.shape[-1] if next_idx is not None else 0
    _check(lib().smoe_route_ext(ctypes.byref(dims_struct(dims)), int(n_tok), _ptr(residual), _ptr(x_out),
                                _ptr(w_router), _ptr(bias), _ptr(topk_idx), _ptr(topk_w), int(n_next),
                                _ptr(next_idx), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))


def moe_decode(dims, x, topk_idx, topk_w, expert_table, residual, ws, stream=None):
    _check(lib().smoe_moe_decode(ctypes.byref(dims_struct(dims)), _ptr(x), _ptr(topk_idx), _ptr(topk_w),
                                 _ptr(expert_table), _ptr(residual), _ptr(ws), ws.numel(), _stream(stream)))


def moe_decode_slots(dims, x, topk_w, blob_ptrs, residual, ws, stream=None):
    arr = (ctypes.c_void_p * len(blob_ptrs))(*[int(p) for p in blob_ptrs])
    _check(lib().smoe_moe_decode_slots(ctypes.byref(dims_struct(dims)), _ptr(x), _ptr(topk_w), arr,
                                       _ptr(residual), _ptr(ws), ws.numel(), _stream(stream)))


def decode_layers(dims, n_layers, residual, w_router, bias, expert_tables, ws, x_rec=None, idx_rec=None,
                  w_rec=None, events=None, stream=None):
    """events: optional list of 2*n_layers raw hipEvent_t handles (ints)."""
    ev = None
    if events is not None:
        assert len(events) == 2 * n_layers
        ev = (ctypes.c_void_p * len(events))(*[int(e) for e in events])
    _check(lib().smoe_decode_layers(ctypes.byref(dims_struct(dims)), int(n_layers), _ptr(residual),
                                    _ptr(w_router), _ptr(bias), _ptr(expert_tables), _ptr(x_rec),
                                    _ptr(idx_rec), _ptr(w_rec), ev, _ptr(ws), ws.numel(), _stream(stream)))


def decode_layers_static(dims, n_layers, residual, w_router, bias, expert_tables, x_rec=None, idx_rec=None,
                         w_rec=None, stream=None):
    """decode_layers on the library's own per-GPU scratch (no workspace)."""
    _check(lib().smoe_decode_layers_static(ctypes.byref(dims_struct(dims)), int(n_layers), _ptr(residual),
                                           _ptr(w_router), _ptr(bias), _ptr(expert_tables), _ptr(x_rec),
                                           _ptr(idx_rec), _ptr(w_rec), _stream(stream)))


def moe_prefill_chunk(dims, x, topk_idx, topk_w, expert_table, residual, union_ids, union_count, offsets,
                      perm, ws, events=None, stream=None):
    """events: optional 4 raw hipEvent_t handles (ints) around the two GEMMs."""
    n_tok = x.shape[0]
    ev = None
    if events is not None:
        assert len(events) == 4
        ev = (ctypes.c_void_p * 4)(*[int(e) for e in events])
    _check(lib().smoe_moe_prefill_chunk(ctypes.byref(dims_struct(dims)), int(n_tok), _ptr(x), _ptr(topk_idx),
                                        _ptr(topk_w), _ptr(expert_table), _ptr(residual), _ptr(union_ids),
                                        _ptr(union_count), _ptr(offsets), _ptr(perm), _ptr(ws), ws.numel(), ev,
                                        _stream(stream)))


class Ring:
    """Host handle of an expert ring (see smoe.h)."""

    def __init__(self, n_slots, n_layers, n_experts, top_k, slot_bytes, slot_stride, vault_layer_ptrs,
                 vault_stride, slab_dev_ptr, copy_stream, log_capacity=0):
        """vault_layer_ptrs: n_layers host addresses, the base of each layer's blobs."""
        assert len(vault_layer_ptrs) == int(n_layers)
        table = (ctypes.c_void_p * int(n_layers))(*[int(p) for p in vault_layer_ptrs])
        desc = SmoeRingDesc(int(n_slots), int(n_layers), int(n_experts), int(top_k), int(slot_bytes),
                            int(slot_stride), table, int(vault_stride), int(slab_dev_ptr),
                            _stream(copy_stream), int(log_capacity))
        h = ctypes.c_void_p(0)
        _check(lib().smoe_ring_create(ctypes.byref(desc), ctypes.byref(h)))
        self.h = h
        self.k = int(top_k)

    def acquire(self, layer, experts, stream=None):
        ex = (ctypes.c_int32 * len(experts))(*[int(e) for e in experts])
        out = (ctypes.c_void_p * len(experts))()
        _check(lib().smoe_ring_acquire(self.h, int(layer), ex, len(experts), out, _stream(stream)))
        return [int(p) for p in out]

    def acquire_table(self, layer, experts, table, stream=None):
        """Acquire ``experts`` (request order) and write the layer's [E] device
        table of blob pointers (NULL for the experts not requested)."""
        ex = (ctypes.c_int32 * len(experts))(*[int(e) for e in experts])
        _check(lib().smoe_ring_acquire_table(self.h, int(layer), ex, len(experts), _ptr(table), _stream(stream)))

    def acquire_routed(self, layer, topk_idx, table, stream=None):
        """Acquire the union of a prefill chunk's routing (device int32
        [n_tok][k]) in first-touch order and write the layer's [E] device
        table; returns the union (host list)."""
        n_tok, k = int(topk_idx.shape[0]), int(topk_idx.shape[1])
        uni = (ctypes.c_int32 * (n_tok * k))()
        nu = ctypes.c_int32(0)
        _check(lib().smoe_ring_acquire_routed(self.h, int(layer), n_tok, k, _ptr(topk_idx), _ptr(table), uni,
                                              ctypes.byref(nu), _stream(stream)))
        return [int(uni[i]) for i in range(nu.value)]

    def prefetch(self, layer, experts, stream=None):
        """Speculative loads of the experts not resident; returns loads issued."""
        ex = (ctypes.c_int32 * max(1, len(experts)))(*[int(e) for e in experts])
        n = ctypes.c_int32(0)
        _check(lib().smoe_ring_prefetch(self.h, int(layer), ex, len(experts), ctypes.byref(n), _stream(stream)))
        return int(n.value)

    def hottest(self, n):
        """[(layer, expert, claims)] of the n most claimed pairs."""
        L = (ctypes.c_int32 * max(1, n))()
        E = (ctypes.c_int32 * max(1, n))()
        C = (ctypes.c_uint64 * max(1, n))()
        m = ctypes.c_int32(0)
        _check(lib().smoe_ring_hottest(self.h, int(n), L, E, C, ctypes.byref(m)))
        return [(int(L[i]), int(E[i]), int(C[i])) for i in range(m.value)]

    def release(self):
        _check(lib().smoe_ring_release(self.h))

    def stats(self):
        v = [ctypes.c_uint64(0) for _ in range(4)]
        _check(lib().smoe_ring_stats(self.h, *[ctypes.byref(x) for x in v]))
        return {"hits": v[0].value, "misses": v[1].value, "evictions": v[2].value, "h2d_bytes": v[3].value}

    def log(self, cap):
        buf = (SmoeRingEvent * int(cap))()
        n = ctypes.c_size_t(0)
        _check(lib().smoe_ring_log(self.h, buf, int(cap), ctypes.byref(n)))
        return [(e.layer, e.rank, e.expert, e.kind, e.slot,
                 None if e.evicted_layer < 0 else (e.evicted_layer, e.evicted_expert))
                for e in buf[: n.value]]

    def destroy(self):
        if self.h:
            _check(lib().smoe_ring_destroy(self.h))
            self.h = None


class PinnedHost:
    """Page-locked host memory from hipHostMalloc (for the ring's vault: fills
    then run as DMA at full PCIe rate).  ``tensor()`` is a CPU uint8 view."""

    def __init__(self, nbytes):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipHostMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t, ctypes.c_uint]
        self._hip.hipHostFree.argtypes = [ctypes.c_void_p]
        p = ctypes.c_void_p(0)
        rc = self._hip.hipHostMalloc(ctypes.byref(p), ctypes.c_size_t(int(nbytes)), 0)
        if rc != 0 or not p.value:
            raise SmoeError(SMOE_ENOMEM, f"hipHostMalloc of {int(nbytes)} bytes failed (hipError {rc})")
        self.ptr = int(p.value)
        self.nbytes = int(nbytes)

    def tensor(self):
        buf = (ctypes.c_uint8 * self.nbytes).from_address(self.ptr)
        return torch.frombuffer(buf, dtype=torch.uint8)

    def free(self):
        if self.ptr:
            self._hip.hipHostFree(ctypes.c_void_p(self.ptr))
            self.ptr = 0
