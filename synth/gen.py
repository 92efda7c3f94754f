"""Seeded synthetic inputs for the routed-expert MoE layer (host side, numpy).

This module only *draws inputs*; it holds none of the layer's arithmetic (no
RMSNorm, routing, dequantisation or FFN).  Both the CPU oracle and the GPU
library are fed from it; ``synth_dev.hip`` is the device twin of the two
integer-only streams (expert codes and scales), written from the same
definitions below so that a 127 GB vault can be drawn on the GPU and any
expert of it redrawn here bit for bit.

Generator (published definition): SplitMix64 (Steele, Lea and Flood,
"Fast splittable pseudorandom number generators", OOPSLA 2014; constants as in
Vigna's public reference code).  A stream is a 64-bit key; its i-th word is
``mix64(key + (i + 1) * GAMMA)`` (mod 2^64), i.e. the i-th output of a
SplitMix64 generator seeded with ``key``.

Stream keys: ``key = mix64(mix64(seed + GAMMA) ^ tag)`` with
``tag = kind << 56 | mat << 48 | layer << 24 | expert``.

Workload shapes follow the pages: Qwen3-30B-A3B and Qwen3-235B-A22B MoE layer
geometry (System Overview, "The Four-Component Architecture" / memory-budget
table: 128 experts, top-8, 94 MoE layers for the 235B model), experts stored as
4-bit codes with a per-chunk affine dequant (Optimizations, "Coalesced GPU
Kernels"), blobs aligned to 16 KB pages ("Rock, Paper, Silicon", the vault).
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK64 = (1 << 64) - 1

KIND_CODES = 1
KIND_SCALES = 2
KIND_ROUTER = 3
KIND_HIDDEN = 4
KIND_BIASPERM = 5
KIND_CODES_Q2 = 6

MAT_GATE, MAT_UP, MAT_DOWN = 0, 1, 2

BLOB_ALIGN = 16384


# --------------------------------------------------------------------------
# SplitMix64
# --------------------------------------------------------------------------
def mix64_int(z: int) -> int:
    """SplitMix64 finaliser on a Python int (mod 2^64)."""
    z &= _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 finaliser on a uint64 array (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, kind: int, layer: int = 0, expert: int = 0, mat: int = 0) -> int:
    assert 0 <= kind < 256 and 0 <= mat < 256 and 0 <= layer < (1 << 24) and 0 <= expert < (1 << 24)
    tag = (kind << 56) | (mat << 48) | (layer << 24) | expert
    return mix64_int(mix64_int(seed + 0x9E3779B97F4A7C15) ^ tag)


def stream_words(key: int, start: int, count: int) -> np.ndarray:
    """Words ``start .. start+count-1`` of the stream ``key`` (uint64)."""
    i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(np.uint64(key) + i * GAMMA)


# --------------------------------------------------------------------------
# bf16 helpers (input encoding only)
# --------------------------------------------------------------------------
def bf16_bits_from_f64(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (round-to-nearest-even, directly from the
    double, no intermediate float32 rounding) and return the 16-bit patterns."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, e = np.frexp(ax)                      # ax = m * 2^e, m in [0.5, 1)
    ulp_exp = np.maximum(e - 8, -133)        # 8 significant bits; bf16 subnormal ulp 2^-133
    q = np.rint(np.ldexp(ax, -ulp_exp))      # exact scaling, round half to even
    r = np.ldexp(q, ulp_exp)
    r = np.where(ax == 0, 0.0, r)
    r = np.copysign(r, x)
    f = r.astype(np.float32)                 # exact: r has <= 8 significant bits
    bits = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return bits


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Uniform / normal draws
# --------------------------------------------------------------------------
def uniform53(words: np.ndarray) -> np.ndarray:
    """Top 53 bits of each word as a double in [0, 1) (exact)."""
    return (words >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal_box_muller(words: np.ndarray) -> np.ndarray:
    """One standard normal deviate per word (Box and Muller, 1958): the high
    32 bits give U1 in (0, 1], the low 32 bits give U2 in [0, 1)."""
    hi = (words >> np.uint64(32)).astype(np.float64)
    lo = (words & np.uint64(0xFFFFFFFF)).astype(np.float64)
    u1 = (hi + 1.0) * (2.0 ** -32)
    u2 = lo * (2.0 ** -32)
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


# --------------------------------------------------------------------------
# Layer geometry and the SMOE-Q4 blob layout
# --------------------------------------------------------------------------
class Dims:
    """Geometry of one routed-expert MoE layer.  ``rms_eps`` is a float32 value
    (the library takes it as float), 1e-6 rounded to float32 by default.
    ``bits`` is the code width of the expert blobs: 4 (SMOE-Q4) or 2
    (SMOE-Q2, the halved vault of the Optimizations page, "Q2 Vaults")."""

    def __init__(self, d_model, d_ff, n_experts, top_k, chunk, norm_topk_prob=True,
                 rms_eps=float(np.float32(1e-6)), bits=4):
        self.d_model = int(d_model)
        self.d_ff = int(d_ff)
        self.n_experts = int(n_experts)
        self.top_k = int(top_k)
        self.chunk = int(chunk)
        self.norm_topk_prob = bool(norm_topk_prob)
        self.rms_eps = float(rms_eps)
        self.bits = int(bits)
        assert self.bits in (2, 4)

    def replace(self, **kw):
        d = dict(self.__dict__)
        d.update(kw)
        return Dims(**d)

    def __repr__(self):
        return (f"Dims(d_model={self.d_model}, d_ff={self.d_ff}, n_experts={self.n_experts}, "
                f"top_k={self.top_k}, chunk={self.chunk}, norm_topk_prob={self.norm_topk_prob}, "
                f"bits={self.bits})")


def blob_sections(dims: Dims) -> dict:
    """Byte offsets of the sections of one expert blob.

    Matrices: gate G[d_ff][d_model], up U[d_ff][d_model], down D[d_model][d_ff].
    Element W[n][k] = scale[n][k // chunk] * q[n][k] + min[n][k // chunk].
    Codes are row-major, 8 / bits per byte, element k of a byte's group in
    bits [bits * k, bits * k + bits) (Q4: the even element in the low nibble;
    Q2: four codes per byte, the first in bits 0..1).
    Per-chunk parameters are (scale, min) bf16 pairs, row-major, scale first.
    Section order: G codes, U codes, D codes, G params, U params, D params.
    """
    d, f, c = dims.d_model, dims.d_ff, dims.chunk
    off = {}
    pos = 0
    for name, rows, cols in (("gate", f, d), ("up", f, d), ("down", d, f)):
        off[name + "_codes"] = pos
        pos += rows * cols * dims.bits // 8
    for name, rows, cols in (("gate", f, d), ("up", f, d), ("down", d, f)):
        off[name + "_params"] = pos
        pos += rows * (cols // c) * 4
    off["bytes"] = pos
    off["stride"] = (pos + BLOB_ALIGN - 1) // BLOB_ALIGN * BLOB_ALIGN
    return off


def _mat_shape(dims: Dims, mat: int):
    if mat == MAT_DOWN:
        return dims.d_model, dims.d_ff
    return dims.d_ff, dims.d_model


def code_words(seed: int, dims: Dims, layer: int, expert: int, mat: int) -> np.ndarray:
    """The matrix's packed code section as stream words: Q4 codes come from
    stream kind 1, Q2 codes from kind 6 (64 / bits codes per word)."""
    rows, cols = _mat_shape(dims, mat)
    per_word = 64 // dims.bits
    assert (rows * cols) % per_word == 0
    kind = KIND_CODES if dims.bits == 4 else KIND_CODES_Q2
    key = stream_key(seed, kind, layer, expert, mat)
    return stream_words(key, 0, rows * cols // per_word)


def unpack_codes(packed: np.ndarray, bits: int) -> np.ndarray:
    """Codes of a packed byte array, element order as in ``blob_sections``."""
    b = np.asarray(packed, dtype=np.uint8)
    per = 8 // bits
    q = np.empty(b.size * per, dtype=np.uint8)
    for j in range(per):
        q[j::per] = (b >> (bits * j)) & ((1 << bits) - 1)
    return q


def pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of ``unpack_codes``."""
    q = np.asarray(q, dtype=np.uint8).reshape(-1)
    per = 8 // bits
    assert q.size % per == 0 and q.max(initial=0) < (1 << bits)
    b = np.zeros(q.size // per, dtype=np.uint8)
    for j in range(per):
        b |= (q[j::per] << (bits * j)).astype(np.uint8)
    return b


def expert_codes(seed: int, dims: Dims, layer: int, expert: int, mat: int) -> np.ndarray:
    """Logical codes q[n][k] (uint8, 0 .. 2^bits - 1) of one matrix."""
    rows, cols = _mat_shape(dims, mat)
    b = code_words(seed, dims, layer, expert, mat).view(np.uint8)
    return unpack_codes(b, dims.bits).reshape(rows, cols)


def expert_params_bits(seed: int, dims: Dims, layer: int, expert: int, mat: int):
    """Per-chunk (scale, min) of one matrix as bf16 bit patterns [rows][cols/chunk].

    scale ~ U(0.002, 0.01) rounded to bf16; min = -2^(bits-1) * scale (exact):
    -8 * scale for Q4, -2 * scale for Q2, so that the mid code is zero."""
    rows, cols = _mat_shape(dims, mat)
    nc = cols // dims.chunk
    key = stream_key(seed, KIND_SCALES, layer, expert, mat)
    u = uniform53(stream_words(key, 0, rows * nc))
    t = 0.008 * u            # two separately rounded double operations
    s = 0.002 + t
    sbits = bf16_bits_from_f64(s)
    mbits = bf16_bits_from_f64(-float(1 << (dims.bits - 1)) * bf16_bits_to_f64(sbits))
    return sbits.reshape(rows, nc), mbits.reshape(rows, nc)


def expert_logical(seed: int, dims: Dims, layer: int, expert: int) -> dict:
    """Codes and per-chunk parameters of all three matrices of one expert."""
    out = {}
    for name, mat in (("gate", MAT_GATE), ("up", MAT_UP), ("down", MAT_DOWN)):
        s, m = expert_params_bits(seed, dims, layer, expert, mat)
        out[name] = {"q": expert_codes(seed, dims, layer, expert, mat), "scale_bits": s, "min_bits": m}
    return out


def pack_blob(seed: int, dims: Dims, layer: int, expert: int) -> np.ndarray:
    """The expert's blob bytes (uint8, padded to the 16 KiB stride)."""
    off = blob_sections(dims)
    blob = np.zeros(off["stride"], dtype=np.uint8)
    for name, mat in (("gate", MAT_GATE), ("up", MAT_UP), ("down", MAT_DOWN)):
        w = code_words(seed, dims, layer, expert, mat).view(np.uint8)
        blob[off[name + "_codes"]: off[name + "_codes"] + w.size] = w
        s, m = expert_params_bits(seed, dims, layer, expert, mat)
        pm = np.empty(s.size * 2, dtype=np.uint16)
        pm[0::2] = s.reshape(-1)
        pm[1::2] = m.reshape(-1)
        pb = pm.view(np.uint8)
        blob[off[name + "_params"]: off[name + "_params"] + pb.size] = pb
    return blob


def pack_logical(dims: Dims, logical: dict) -> np.ndarray:
    """Blob bytes for arbitrary logical codes/params (used to build hand-made
    experts in tests: duplicated experts, zero experts, ...)."""
    off = blob_sections(dims)
    blob = np.zeros(off["stride"], dtype=np.uint8)
    for name in ("gate", "up", "down"):
        b = pack_codes(logical[name]["q"], dims.bits)
        blob[off[name + "_codes"]: off[name + "_codes"] + b.size] = b
        s = np.asarray(logical[name]["scale_bits"], dtype=np.uint16).reshape(-1)
        m = np.asarray(logical[name]["min_bits"], dtype=np.uint16).reshape(-1)
        pm = np.empty(s.size * 2, dtype=np.uint16)
        pm[0::2] = s
        pm[1::2] = m
        pb = pm.view(np.uint8)
        blob[off[name + "_params"]: off[name + "_params"] + pb.size] = pb
    return blob


# --------------------------------------------------------------------------
# Router weights, hidden states, logit bias
# --------------------------------------------------------------------------
def router_bits(seed: int, dims: Dims, layer: int, std: float = 0.02) -> np.ndarray:
    """Router gate weights [E][d_model] ~ N(0, std^2), as bf16 bit patterns."""
    key = stream_key(seed, KIND_ROUTER, layer)
    z = normal_box_muller(stream_words(key, 0, dims.n_experts * dims.d_model))
    return bf16_bits_from_f64(std * z).reshape(dims.n_experts, dims.d_model)


def normal_vector(seed: int, stream: int, n: int, sub: int = 0) -> np.ndarray:
    """A standard-normal float64 vector, stream ``stream`` (e.g. a step index)."""
    key = stream_key(seed, KIND_HIDDEN, stream, sub)
    return normal_box_muller(stream_words(key, 0, n))


def hidden_bf16(seed: int, stream: int, n: int, sub: int = 0) -> np.ndarray:
    """A hidden state ~N(0, 1) rounded to bf16, widened to float32."""
    return bf16_bits_to_f64(bf16_bits_from_f64(normal_vector(seed, stream, n, sub))).astype(np.float32)


def zipf_bias(seed: int, dims: Dims, layer: int, s: float = 1.1) -> np.ndarray:
    """Per-expert logit bias -s * ln(rank), rank a seeded permutation of 1..E
    (Fisher-Yates driven by the stream).  Returned as float32."""
    E = dims.n_experts
    key = stream_key(seed, KIND_BIASPERM, layer)
    words = stream_words(key, 0, E)
    perm = list(range(E))
    for i in range(E - 1, 0, -1):
        j = int(words[i] % np.uint64(i + 1))
        perm[i], perm[j] = perm[j], perm[i]
    rank = np.asarray(perm, dtype=np.float64) + 1.0
    return (-s * np.log(rank)).astype(np.float32)


def markov_hidden(seed: int, n_steps: int, n: int, keep: float = 0.7, fresh: float = 0.3,
                  lane: int = 0) -> np.ndarray:
    """Hidden states h_t = keep * h_{t-1} + fresh * z_t, h_0 = z_0 (float64
    recursion, rounded to float32 at the end).  Shape [n_steps][n].  ``lane``
    selects an independent chain (e.g. one per layer)."""
    out = np.empty((n_steps, n), dtype=np.float32)
    h = None
    for t in range(n_steps):
        z = normal_vector(seed, t, n, sub=1 + lane)
        h = z if h is None else keep * h + fresh * z
        out[t] = h.astype(np.float32)
    return out
