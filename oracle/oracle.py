"""CPU oracle for the routed-expert MoE layer -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 numpy.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; the product path (the
HIP library and its Python binding) never does.  It shares no code with the
GPU library: it reads logical inputs (4-bit codes, bf16 bit patterns, float
residuals) and implements every step from its definition.

What it computes, and where the pages define it
-----------------------------------------------
Sources are three pages: "Optimizations" (docs.s-moe.com, v1), "System
Overview" (docs.s-moe.com, v1) and the S-MoE diary feed.

* RMSNorm of the residual into the bf16 router / expert input -- the per-layer
  norm that "The Dense Ceiling -- GPU-Resident Epilogue" (Optimizations) moves
  next to the router gate.  Gain 1, eps 1e-6 (reading: the pages give neither).
* Exact router: an E x d_model gate matvec on the actual hidden state (no
  predictor), then top-k selection and Qwen3's norm_topk_prob weighting
  (Optimizations, "Routing Is Exact"; System Overview, per-token step table).
  Qwen3's definition: softmax over all E logits, keep the k largest, and when
  norm_topk_prob is set divide the kept probabilities by their sum.
* Fused SMOE-Q4 expert FFN: per-chunk affine dequant, gate and up on the same
  input, SwiGLU, down projection, and the gate-weighted sum of the k expert
  outputs added into the residual (Optimizations, "Coalesced GPU Kernels";
  System Overview, step table, "Metal Kernel" row).  The SMOE-Q2 vault of
  the Optimizations page ("Q2 Vaults -- the Next 2x") uses the same affine
  dequant with 2-bit codes; the oracle reads logical codes, so only their
  range (0..3 instead of 0..15) differs.
* Layer-major prefill: the distinct experts of a chunk form a union that is
  streamed once (Optimizations, "Prefill Reads Each Expert Once"); the union
  is listed in first-touch order because that section has each expert
  dispatched as soon as some token of the chunk first selects it.
* The LRU expert ring: hit = same (layer, expert) already resident, zero bytes
  read; lazy least-recently-used eviction that never evicts a slot the current
  layer holds (Optimizations, "The Ring Is an LRU Cache").

Readings where the pages are silent are listed in the design notes and in the
docstrings below.  Every function here is pinned by tests under tests/ against
closed forms, brute force or textbook routines; none is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np


# ---------------------------------------------------------------------------
# bf16 encode / decode
# ---------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """Value of each bf16 bit pattern (the upper half of an IEEE binary32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_round(x) -> np.ndarray:
    """Nearest bf16 value to each double, ties to the even significand.

    bf16 keeps 8 significant bits; below 2^-126 the spacing is fixed at
    2^-133 (subnormals).  Computed by bracketing |x| between two neighbouring
    representable values and picking the nearer; every step is exact in
    float64.  Returns (values as float64, bit patterns as uint16)."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    # log2 can be off by one near powers of two: fix the binade exactly.
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > ax, e - 1, e)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= ax, e + 1, e)
    spacing_exp = np.maximum(e - 7, -133).astype(np.int64)
    spacing = np.ldexp(1.0, spacing_exp)
    n_lo = np.floor(ax / spacing)                 # exact: power-of-two scaling
    lo = n_lo * spacing
    hi = lo + spacing
    d_lo = ax - lo
    d_hi = hi - ax
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (np.mod(n_lo, 2) == 1))
    r = np.where(pick_hi, hi, lo)
    r = np.where(ax == 0, 0.0, r)
    r = np.where(r > 3.3895313892515355e38, np.inf, r)   # beyond the largest bf16: overflow
    r = np.copysign(r, x)
    bits = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return r, bits


# ---------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------
def rmsnorm_bf16(r, eps: float = 1e-6):
    """x = bf16( r / sqrt(mean(r^2) + eps) ) for one residual vector (gain 1).

    Returns (x values float64, x bf16 bits)."""
    r = np.asarray(r, dtype=np.float64)
    ms = np.sum(r * r) / r.size
    return bf16_round(r / math.sqrt(ms + eps))


# ---------------------------------------------------------------------------
# Router
# ---------------------------------------------------------------------------
def router_logits(w_router_bits, x, bias=None) -> np.ndarray:
    """l_e = sum_j W[e, j] x_j (+ b_e), float64.  Each product of two bf16
    values is exact in float64."""
    w = bf16_to_f64(w_router_bits)
    l = w @ np.asarray(x, dtype=np.float64)
    if bias is not None:
        l = l + np.asarray(bias, dtype=np.float64)
    return l


def select_topk(logits, k: int, norm_topk_prob: bool = True):
    """Exact top-k and mixing weights, Qwen3 style.

    Order: a full stable sort on (-logit, expert index) -- equal logits go to the
    lower index -- and the first k are taken, in rank order.
    Weights: p = softmax over all E logits; w_r = p[e_r], divided by
    sum_r p[e_r] when norm_topk_prob is set.  Returns (idx int list, w float64)."""
    l = np.asarray(logits, dtype=np.float64)
    E = l.size
    order = sorted(range(E), key=lambda e: (-l[e], e))
    idx = order[:k]
    p = np.exp(l - l.max())
    p = p / p.sum()
    w = p[idx]
    if norm_topk_prob:
        w = w / w.sum()
    return idx, w


# ---------------------------------------------------------------------------
# SMOE-Q4 / SMOE-Q2 expert
# ---------------------------------------------------------------------------
def dequant(q, scale_bits, min_bits, chunk: int) -> np.ndarray:
    """W[n][k] = scale[n][k // chunk] * q[n][k] + min[n][k // chunk] (float64),
    for codes of any width (Q4: 0..15, Q2: 0..3)."""
    q = np.asarray(q, dtype=np.float64)
    s = np.repeat(bf16_to_f64(scale_bits), chunk, axis=1)
    m = np.repeat(bf16_to_f64(min_bits), chunk, axis=1)
    assert s.shape == q.shape
    return s * q + m


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def expert_ffn(expert: dict, x, chunk: int, return_h: bool = False):
    """One SwiGLU expert on input x: y = D (silu(G x) * (U x))."""
    x = np.asarray(x, dtype=np.float64)
    G = dequant(expert["gate"]["q"], expert["gate"]["scale_bits"], expert["gate"]["min_bits"], chunk)
    g = G @ x
    del G
    U = dequant(expert["up"]["q"], expert["up"]["scale_bits"], expert["up"]["min_bits"], chunk)
    u = U @ x
    del U
    h = silu(g) * u
    D = dequant(expert["down"]["q"], expert["down"]["scale_bits"], expert["down"]["min_bits"], chunk)
    y = D @ h
    if return_h:
        return y, h
    return y


def moe_layer(residual, w_router_bits, experts, dims, bias=None, return_h: bool = False, ffn=None):
    """One routed-MoE layer on one token.

    ``experts`` maps an expert index to its logical codes/params (only the
    selected ones are touched, so a lazy mapping works).  ``ffn``, if given,
    is called as ffn(e, x, x_bits) in place of expert_ffn(experts[e], x, chunk)
    (a caller may memoise expert outputs; it must return the same values).
    Returns a dict with x (values, bits), logits, idx, w, y (the MoE output,
    float64) and r_out = residual + y."""
    x, xbits = rmsnorm_bf16(residual, dims.rms_eps)
    l = router_logits(w_router_bits, x, bias)
    idx, w = select_topk(l, dims.top_k, dims.norm_topk_prob)
    y = np.zeros(dims.d_model, dtype=np.float64)
    hs = []
    for r, e in enumerate(idx):                       # rank order
        if ffn is not None and not return_h:
            y = y + w[r] * ffn(e, x, xbits)
            continue
        out = expert_ffn(experts[e], x, dims.chunk, return_h=return_h)
        if return_h:
            out, h = out
            hs.append(h)
        y = y + w[r] * out
    res = {"x": x, "x_bits": xbits, "logits": l, "idx": idx, "w": w, "y": y,
           "r_out": np.asarray(residual, dtype=np.float64) + y}
    if return_h:
        res["h"] = hs
    return res


# ---------------------------------------------------------------------------
# Layer-major prefill: union of a chunk's experts
# ---------------------------------------------------------------------------
def expert_union(idx):
    """Union of the experts a chunk routes to, in first-touch order.

    ``idx`` is [T][k] (rank order per token).  Scanning t = 0..T-1 and then
    r = 0..k-1, an expert joins the union the first time it is seen.  For union
    member u: count n_u, exclusive offset o_u in union order, and its token
    list in t-ascending order, each entry encoded as t * k + r.
    Returns (union ids, counts, offsets [|U|+1], perm [T*k])."""
    idx = [list(map(int, row)) for row in idx]
    T = len(idx)
    k = len(idx[0]) if T else 0
    union = []
    members = {}
    for t in range(T):
        for r in range(k):
            e = idx[t][r]
            if e not in members:
                members[e] = []
                union.append(e)
            members[e].append(t * k + r)
    counts = [len(members[e]) for e in union]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    perm = []
    for e in union:
        perm.extend(members[e])
    return union, counts, offsets, perm


def prefill_chunk(residuals, w_router_bits, experts, dims, bias=None):
    """Layer-major prefill of one chunk through one layer: every token is
    routed exactly and gets the same MoE output as in decode; the union says
    which experts the chunk reads (each once)."""
    outs = [moe_layer(r, w_router_bits, experts, dims, bias) for r in residuals]
    union, counts, offsets, perm = expert_union([o["idx"] for o in outs])
    return {"tokens": outs, "union": union, "counts": counts, "offsets": offsets, "perm": perm}


# ---------------------------------------------------------------------------
# The LRU expert ring
# ---------------------------------------------------------------------------
HIT, MISS, PREFETCH = 0, 1, 2


class LruRing:
    """Step-by-step simulation of the expert ring's slot policy.

    State per slot: key (layer, expert) or empty, last-use tick, pinned flag.
    A global tick advances by one per request.  Protocol per layer: the
    previous layer's pins are dropped (``release``), then the k routed experts
    are requested in rank order (``acquire``):
      * resident key -> HIT: tick := now, pinned; zero bytes move;
      * otherwise MISS: the lowest-index empty slot, else the unpinned
        occupied slot with the smallest tick (evicted), is loaded: key set,
        tick := now, pinned.
    Reading: the section says new loads get a fresh tick and also calls the
    policy least-recently-used; here every request, hit or load, stamps the
    slot (true LRU).  Slots are
    never wiped; retention spans tokens."""

    def __init__(self, n_slots: int):
        self.n = int(n_slots)
        self.keys = [None] * self.n
        self.tick = np.full(self.n, -1, dtype=np.int64)
        self.pinned = np.zeros(self.n, dtype=bool)
        self.now = 0
        self.where = {}
        self.hits = self.misses = self.evictions = 0
        self.prefetches = 0

    def release(self):
        self.pinned[:] = False

    def acquire(self, layer: int, experts):
        """Returns events (layer, rank, expert, HIT|MISS, slot, evicted key or None)."""
        events = []
        for r, e in enumerate(experts):
            key = (int(layer), int(e))
            if key in self.where:
                s = self.where[key]
                kind, evicted = HIT, None
                self.hits += 1
            else:
                empty = [i for i in range(self.n) if self.keys[i] is None]
                if empty:
                    s, evicted = empty[0], None
                else:
                    cand = np.where(~self.pinned, self.tick, np.iinfo(np.int64).max)
                    s = int(np.argmin(cand))
                    if self.pinned[s]:
                        raise RuntimeError("no unpinned slot")
                    evicted = self.keys[s]
                    del self.where[evicted]
                    self.evictions += 1
                self.keys[s] = key
                self.where[key] = s
                kind = MISS
                self.misses += 1
            self.tick[s] = self.now
            self.pinned[s] = True
            self.now += 1
            events.append((key[0], r, key[1], kind, s, evicted))
        return events

    def _victim(self):
        """Lowest-index empty slot, else the unpinned slot with the oldest
        tick; None when every slot is pinned."""
        for i in range(self.n):
            if self.keys[i] is None:
                return i
        cand = np.where(~self.pinned, self.tick, np.iinfo(np.int64).max)
        s = int(np.argmin(cand))
        return None if self.pinned[s] else s

    def prefetch(self, layer: int, experts):
        """Speculative loads (not demand): each expert not resident is loaded
        into the victim slot the same policy picks, with a fresh tick and no
        pin; a resident expert is left untouched (no tick).  Stops when every
        slot is pinned (a bet never displaces the current acquisition).
        Returns one PREFETCH event per load."""
        events = []
        for r, e in enumerate(experts):
            key = (int(layer), int(e))
            if key in self.where:
                continue
            s = self._victim()
            if s is None:
                break
            evicted = self.keys[s]
            if evicted is not None:
                del self.where[evicted]
                self.evictions += 1
            self.keys[s] = key
            self.where[key] = s
            self.tick[s] = self.now
            self.now += 1
            self.prefetches += 1
            events.append((key[0], r, key[1], PREFETCH, s, evicted))
        return events


def ring_trace(routing, n_slots: int):
    """Simulate the ring over a decode trace.  ``routing[t][L]`` is the rank-
    ordered expert list of token t at layer L.  Returns the event list and
    (hits, misses, evictions)."""
    ring = LruRing(n_slots)
    events = []
    for t, layers in enumerate(routing):
        for L, experts in enumerate(layers):
            ring.release()
            events.extend((t,) + ev for ev in ring.acquire(L, experts))
    return events, (ring.hits, ring.misses, ring.evictions)
