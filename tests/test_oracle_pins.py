"""Pins of the CPU oracle against facts that do not come from the oracle itself:
closed forms, hand-derived small cases, brute force and library routines.

The pages print no worked numeric example for this layer, so every pin here is
a closed form, an invariant or an independent computation."""
import bisect
import itertools
import math
from collections import OrderedDict
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

# ---------------------------------------------------------------------------
# bf16 rounding
# ---------------------------------------------------------------------------
_ALL_BF16 = None


def _all_finite_bf16():
    global _ALL_BF16
    if _ALL_BF16 is None:
        bits = np.arange(0, 0x7F80, dtype=np.uint32)          # +0 .. largest finite
        vals = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
        _ALL_BF16 = (vals.tolist(), bits.tolist())
    return _ALL_BF16


def _nearest_bf16_bruteforce(x: float) -> float:
    """Nearest finite bf16 by exact rational distance, ties to even pattern."""
    vals, bits = _all_finite_bf16()
    ax = abs(x)
    i = bisect.bisect_left(vals, ax)
    cands = [j for j in (i - 1, i, i + 1) if 0 <= j < len(vals)]
    best = None
    for j in cands:
        dist = abs(Fraction(vals[j]) - Fraction(ax))
        key = (dist, bits[j] & 1)
        if best is None or key < best[0]:
            best = (key, vals[j])
    return math.copysign(best[1], x)


def test_bf16_round_hand_cases():
    # 1 + 2^-8 lies exactly half-way between 1 and 1 + 2^-7: ties to the even significand (1).
    # 1 + 3*2^-8 lies half-way between 1 + 2^-7 (odd) and 1 + 2^-6 (even): rounds up.
    v, b = oracle.bf16_round([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.0, 2 ** -130, 0.0, -0.0, 1e39])
    assert v[0] == 1.0 and b[0] == 0x3F80
    assert v[1] == 1.0
    assert v[2] == 1 + 2 ** -6 and b[2] == 0x3F82
    assert v[3] == -2.0 and b[3] == 0xC000
    assert v[4] == 2 ** -130 and b[4] == 0x0008           # subnormal, exact
    assert v[5] == 0.0 and b[5] == 0 and b[6] == 0x8000
    assert math.isinf(v[7]) and b[7] == 0x7F80


def test_bf16_round_brute_force():
    rng = np.random.default_rng(5)
    xs = np.concatenate([
        rng.standard_normal(600) * 3.0,
        rng.standard_normal(200) * 1e-3,
        np.ldexp(rng.uniform(1, 2, 100), rng.integers(-140, -120, 100)),   # around the subnormal edge
        np.array([1 + 2 ** -8 + 2 ** -40, 1 + 2 ** -8 - 2 ** -40, 3.0 * 2 ** -9]),
    ])
    got, _ = oracle.bf16_round(xs)
    for x, g in zip(xs.tolist(), got.tolist()):
        assert g == _nearest_bf16_bruteforce(x), x


def test_bf16_round_matches_torch_on_float32_inputs():
    # For inputs that are float32 values the double is exact, so torch's
    # float32 -> bfloat16 conversion (round to nearest even) is a single rounding.
    rng = np.random.default_rng(7)
    f = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    _, bits = oracle.bf16_round(f.astype(np.float64))
    tb = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, tb)


def test_bf16_round_fixed_points():
    bits = np.arange(0, 0x7F80, 97, dtype=np.uint16)
    v = oracle.bf16_to_f64(bits)
    r, b = oracle.bf16_round(v)
    assert np.array_equal(b, bits) and np.array_equal(r, v)


# ---------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------
def test_rmsnorm_constant_vector_closed_form():
    # r = c * ones: mean(r^2) = c^2, x = c / sqrt(c^2 + eps) for every element.
    for c in (3.0, -0.25, 1e-4):
        x, _ = oracle.rmsnorm_bf16(np.full(64, c), eps=1e-6)
        expect, _ = oracle.bf16_round(np.array([c / math.sqrt(c * c + 1e-6)]))
        assert np.all(x == expect[0])


def test_rmsnorm_power_of_two_scale_invariance():
    rng = np.random.default_rng(1)
    r = rng.standard_normal(512)
    a, ab = oracle.rmsnorm_bf16(r, eps=0.0)
    b, bb = oracle.rmsnorm_bf16(8.0 * r, eps=0.0)
    assert np.array_equal(ab, bb)


def test_rmsnorm_matches_torch_rms_norm_before_rounding():
    rng = np.random.default_rng(2)
    r = rng.standard_normal(1000) * 2.5
    t = torch.nn.functional.rms_norm(torch.from_numpy(r)[None], (1000,), eps=1e-6)[0].numpy()
    x, _ = oracle.rmsnorm_bf16(r, eps=1e-6)
    tr, _ = oracle.bf16_round(t)
    # torch multiplies by rsqrt; the oracle divides by sqrt: the doubles agree to
    # a few ulps, so at most a rare bf16 tie-break differs.
    assert np.mean(x == tr) > 0.999
    assert np.max(np.abs(x - t) / np.maximum(np.abs(t), 1e-30)) <= 2 ** -8


# ---------------------------------------------------------------------------
# Router: logits, top-k, weights
# ---------------------------------------------------------------------------
def test_router_logits_exact_rational():
    rng = np.random.default_rng(3)
    E, d = 6, 48
    wb = synth.bf16_bits_from_f64(rng.standard_normal((E, d)) * 0.02)
    _, xb = oracle.bf16_round(rng.standard_normal(d))
    x = oracle.bf16_to_f64(xb)
    w = oracle.bf16_to_f64(wb)
    got = oracle.router_logits(wb, x)
    for e in range(E):
        exact = sum(Fraction(float(w[e, j])) * Fraction(float(x[j])) for j in range(d))
        assert abs(Fraction(float(got[e])) - exact) <= abs(exact) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 80)


def _topk_by_repeated_argmax(l, k):
    l = list(map(float, l))
    taken = []
    for _ in range(k):
        best = None
        for e, v in enumerate(l):
            if e in taken:
                continue
            if best is None or v > l[best]:      # strict: the lower index wins ties
                best = e
        taken.append(best)
    return taken


def test_topk_matches_repeated_argmax_and_torch():
    rng = np.random.default_rng(4)
    for E, k in ((16, 4), (128, 8), (128, 1), (8, 8)):
        for _ in range(20):
            l = rng.standard_normal(E)
            idx, _ = oracle.select_topk(l, k)
            assert idx == _topk_by_repeated_argmax(l, k)
            tv, ti = torch.topk(torch.from_numpy(l), k)
            assert idx == ti.tolist()


def test_topk_tie_break_lower_index_first():
    l = np.array([0.5, 1.0, 0.25, 1.0, 1.0, -3.0])
    idx, w = oracle.select_topk(l, 4)
    assert idx == [1, 3, 4, 0]
    assert w[0] == w[1] == w[2]


def test_weights_sum_to_one_and_descend():
    rng = np.random.default_rng(6)
    for _ in range(50):
        l = rng.standard_normal(128) * 1.3
        idx, w = oracle.select_topk(l, 8, True)
        assert abs(w.sum() - 1.0) <= 1e-12
        assert np.all(np.diff(w) <= 0)


def test_weights_k_equals_E_is_full_softmax():
    rng = np.random.default_rng(8)
    l = rng.standard_normal(16)
    idx, w = oracle.select_topk(l, 16, True)
    sm = torch.softmax(torch.from_numpy(l), 0).numpy()
    assert np.allclose(w, sm[idx], rtol=1e-13, atol=0)


def test_weights_norm_topk_equals_softmax_over_selected_logits():
    rng = np.random.default_rng(9)
    l = rng.standard_normal(128)
    idx, w = oracle.select_topk(l, 8, True)
    sm = torch.softmax(torch.from_numpy(l[idx]), 0).numpy()
    assert np.allclose(w, sm, rtol=1e-13, atol=0)


def test_weights_without_renormalisation_two_expert_closed_form():
    # Two experts, k = 1, no renormalisation: w = sigmoid(l1 - l2).
    for l1, l2 in ((0.3, -0.2), (2.0, 1.5), (-1.0, -4.0)):
        idx, w = oracle.select_topk(np.array([l1, l2]), 1, False)
        assert idx == [0]
        assert abs(w[0] - 1.0 / (1.0 + math.exp(-(l1 - l2)))) <= 1e-15
    idx, w = oracle.select_topk(np.array([0.3, 0.9]), 1, True)
    assert idx == [1] and w[0] == 1.0


def test_weights_shift_invariant():
    rng = np.random.default_rng(10)
    l = rng.standard_normal(128)
    i1, w1 = oracle.select_topk(l, 8, True)
    i2, w2 = oracle.select_topk(l + 0.75, 8, True)
    assert i1 == i2 and np.allclose(w1, w2, rtol=1e-14)


def test_bias_shapes_selection():
    l = np.array([1.0, 0.9, 0.8, 0.7])
    b = np.array([-1.0, 0.0, 0.0, 0.5])
    x = np.zeros(4)
    # W = identity rows scaled so that logits equal l (exact in bf16 for these values)
    wbits = synth.bf16_bits_from_f64(np.eye(4))
    l2 = oracle.router_logits(wbits, l, b)
    assert np.array_equal(l2, l + b)
    idx, _ = oracle.select_topk(l2, 2)
    assert idx == [3, 1]


# ---------------------------------------------------------------------------
# Dequant and the expert FFN
# ---------------------------------------------------------------------------
def _hand_expert():
    """d_model 4, d_ff 2, chunk 2.  Dequantised matrices derived by hand."""
    b = lambda v: synth.bf16_bits_from_f64(np.asarray(v, dtype=np.float64))
    return {
        # G row0: [0.5*8-4, 0.5*9-4, 0.25*0-2, 0.25*15-2] = [0, 0.5, -2, 1.75]
        # G row1: [1*3-8, 1*8-8, 0.125*8-1, 0.125*12-1] = [-5, 0, 0, 0.5]
        "gate": {"q": np.array([[8, 9, 0, 15], [3, 8, 8, 12]], dtype=np.uint8),
                 "scale_bits": b([[0.5, 0.25], [1.0, 0.125]]),
                 "min_bits": b([[-4.0, -2.0], [-8.0, -1.0]])},
        # U row0: [1, 0, 0, 0]; U row1: [0, 0, -4, 0]
        "up": {"q": np.array([[10, 8, 8, 8], [8, 8, 4, 8]], dtype=np.uint8),
               "scale_bits": b([[0.5, 0.5], [0.5, 1.0]]),
               "min_bits": b([[-4.0, -4.0], [-4.0, -8.0]])},
        # D rows: [1, 0], [0, 1], [0.5, 0.5], [0.4375, -0.4375]
        "down": {"q": np.array([[9, 8], [8, 10], [0, 0], [15, 1]], dtype=np.uint8),
                 "scale_bits": b([[1.0], [0.5], [0.25], [0.0625]]),
                 "min_bits": b([[-8.0], [-4.0], [0.5], [-0.5]])},
    }


def test_dequant_hand_example():
    ex = _hand_expert()
    G = oracle.dequant(ex["gate"]["q"], ex["gate"]["scale_bits"], ex["gate"]["min_bits"], 2)
    assert G.tolist() == [[0, 0.5, -2, 1.75], [-5, 0, 0, 0.5]]
    U = oracle.dequant(ex["up"]["q"], ex["up"]["scale_bits"], ex["up"]["min_bits"], 2)
    assert U.tolist() == [[1, 0, 0, 0], [0, 0, -4, 0]]
    D = oracle.dequant(ex["down"]["q"], ex["down"]["scale_bits"], ex["down"]["min_bits"], 2)
    assert D.tolist() == [[1, 0], [0, 1], [0.5, 0.5], [0.4375, -0.4375]]


def test_expert_ffn_hand_example_closed_form():
    ex = _hand_expert()
    x = np.array([1.0, 2.0, 0.5, -1.0])
    # g = G x = [-1.75, -5.5]; u = U x = [1, -2]; h = silu(g) * u
    h0 = -1.75 / (1 + math.exp(1.75)) * 1.0
    h1 = -5.5 / (1 + math.exp(5.5)) * -2.0
    expect = [h0, h1, 0.5 * (h0 + h1), 0.4375 * (h0 - h1)]
    y = oracle.expert_ffn(ex, x, 2)
    assert np.allclose(y, expect, rtol=1e-15, atol=1e-17)


def test_dequant_zero_code_and_round_trip():
    dims = synth.Dims(64, 32, 4, 2, 32)
    for mat in (synth.MAT_GATE, synth.MAT_DOWN):
        q = synth.expert_codes(1337, dims, 0, 1, mat)
        sb, mb = synth.expert_params_bits(1337, dims, 0, 1, mat)
        W = oracle.dequant(q, sb, mb, dims.chunk)
        s = np.repeat(oracle.bf16_to_f64(sb), dims.chunk, 1)
        m = np.repeat(oracle.bf16_to_f64(mb), dims.chunk, 1)
        assert np.all(W[q == 8] == 0.0)                         # min = -8 * scale
        assert np.array_equal(np.rint((W - m) / s).astype(np.uint8), q)  # requantise
        # exact in float32 as well: s*q has <= 12 significant bits
        w32 = (s.astype(np.float32) * q.astype(np.float32)) + m.astype(np.float32)
        assert np.array_equal(w32.astype(np.float64), W)


def test_dequant_quantisation_error_bound():
    # Quantising a random chunk with this affine grid and dequantising is
    # within half a step of the value.
    rng = np.random.default_rng(11)
    v = rng.uniform(-0.05, 0.05, (8, 64))
    s = (v.max(1) - v.min(1)) / 15.0
    mn = v.min(1)
    sb = synth.bf16_bits_from_f64(s)[:, None]
    mb = synth.bf16_bits_from_f64(mn)[:, None]
    sv = oracle.bf16_to_f64(sb)
    mv = oracle.bf16_to_f64(mb)
    q = np.clip(np.rint((v - mv) / sv), 0, 15).astype(np.uint8)
    W = oracle.dequant(q, sb, mb, 64)
    inside = (v >= mv) & (v <= mv + 15 * sv)
    bound = np.broadcast_to(sv / 2 + 1e-15, v.shape)
    assert np.all(np.abs(W - v)[inside] <= bound[inside])


def _dense_swiglu_torch(ex, x, chunk):
    """Dense SwiGLU FFN via torch: dequantised weights built with torch ops,
    torch's silu, float64."""
    def W(m):
        q = torch.from_numpy(ex[m]["q"].astype(np.float64))
        s = torch.from_numpy(oracle.bf16_to_f64(ex[m]["scale_bits"])).repeat_interleave(chunk, 1)
        mn = torch.from_numpy(oracle.bf16_to_f64(ex[m]["min_bits"])).repeat_interleave(chunk, 1)
        return torch.addcmul(mn, s, q)
    xt = torch.from_numpy(np.asarray(x, dtype=np.float64))
    h = torch.nn.functional.silu(W("gate") @ xt) * (W("up") @ xt)
    return (W("down") @ h).numpy()


def _tiny_stack(seed=1337, dims=None, layer=0):
    dims = dims or synth.Dims(256, 128, 16, 4, 32)
    experts = {e: synth.expert_logical(seed, dims, layer, e) for e in range(dims.n_experts)}
    wr = synth.router_bits(seed, dims, layer)
    return dims, experts, wr


def test_single_expert_weight_one_is_dense_swiglu():
    dims, experts, wr = _tiny_stack()
    d1 = dims.replace(top_k=1)
    r = synth.hidden_bf16(1337, 0, dims.d_model).astype(np.float64)
    out = oracle.moe_layer(r, wr, experts, d1)
    assert out["w"].tolist() == [1.0]
    dense = _dense_swiglu_torch(experts[out["idx"][0]], out["x"], dims.chunk)
    assert np.allclose(out["y"], dense, rtol=1e-12, atol=1e-14)
    assert np.array_equal(out["r_out"], r + out["y"])


def test_zero_input_gives_zero_output():
    dims, experts, wr = _tiny_stack()
    y = oracle.expert_ffn(experts[3], np.zeros(dims.d_model), dims.chunk)
    assert np.all(y == 0.0)


def test_duplicated_expert_split_weights():
    # Experts 0 and 1 identical, router rows 0 and 1 identical -> a forced tie,
    # both selected with equal weight; the mix equals the single expert.
    dims, experts, wr = _tiny_stack()
    experts = dict(experts)
    experts[1] = experts[0]
    wr = wr.copy()
    wr[1] = wr[0]
    # make rows 0/1 the clear winners
    wr[0] = wr[1] = synth.bf16_bits_from_f64(np.full(dims.d_model, 0.05))
    r = np.abs(synth.hidden_bf16(1337, 3, dims.d_model).astype(np.float64))
    out2 = oracle.moe_layer(r, wr, experts, dims.replace(top_k=2))
    out1 = oracle.moe_layer(r, wr, experts, dims.replace(top_k=1))
    assert out2["idx"] == [0, 1] and out2["w"][0] == out2["w"][1] == 0.5
    assert np.allclose(out2["y"], out1["y"], rtol=1e-14, atol=1e-16)


def test_expert_relabelling_invariance():
    dims, experts, wr = _tiny_stack()
    perm = np.random.default_rng(12).permutation(dims.n_experts)
    experts2 = {int(perm[e]): experts[e] for e in range(dims.n_experts)}
    wr2 = np.empty_like(wr)
    wr2[perm] = wr
    r = synth.hidden_bf16(1337, 5, dims.d_model).astype(np.float64)
    a = oracle.moe_layer(r, wr, experts, dims)
    b = oracle.moe_layer(r, wr2, experts2, dims)
    assert [int(perm[e]) for e in a["idx"]] == b["idx"]
    assert np.allclose(a["y"], b["y"], rtol=1e-13, atol=1e-15)


def test_expert_order_permutation_gives_same_mix():
    dims, experts, wr = _tiny_stack()
    r = synth.hidden_bf16(1337, 6, dims.d_model).astype(np.float64)
    a = oracle.moe_layer(r, wr, experts, dims)
    ys = [oracle.expert_ffn(experts[e], a["x"], dims.chunk) for e in a["idx"]]
    rev = sum(a["w"][i] * ys[i] for i in reversed(range(len(ys))))
    assert np.allclose(a["y"], rev, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------------------
# SMOE-Q2 (2-bit codes, the same per-chunk affine dequant)
# ---------------------------------------------------------------------------
def _hand_expert_q2():
    """d_model 4, d_ff 2, chunk 2, codes 0..3.  Dequantised matrices by hand."""
    b = lambda v: synth.bf16_bits_from_f64(np.asarray(v, dtype=np.float64))
    return {
        # G row0: [0.5*2-1, 0.5*3-1, 1*0-2, 1*3-2] = [0, 0.5, -2, 1]
        # G row1: [2*1-4, 2*2-4, 0.25*2-0.5, 0.25*0-0.5] = [-2, 0, 0, -0.5]
        "gate": {"q": np.array([[2, 3, 0, 3], [1, 2, 2, 0]], dtype=np.uint8),
                 "scale_bits": b([[0.5, 1.0], [2.0, 0.25]]),
                 "min_bits": b([[-1.0, -2.0], [-4.0, -0.5]])},
        # U row0: [1, 0, 0, 0]; U row1: [0, 0, -4, 0]
        "up": {"q": np.array([[3, 2, 2, 2], [2, 2, 0, 2]], dtype=np.uint8),
               "scale_bits": b([[1.0, 1.0], [1.0, 2.0]]),
               "min_bits": b([[-2.0, -2.0], [-2.0, -4.0]])},
        # D rows: [1, 0], [0, 1], [0.5, 0.5], [0.5, -0.5]
        "down": {"q": np.array([[3, 2], [2, 3], [2, 2], [3, 1]], dtype=np.uint8),
                 "scale_bits": b([[1.0], [1.0], [0.25], [0.5]]),
                 "min_bits": b([[-2.0], [-2.0], [0.0], [-1.0]])},
    }


def test_q2_dequant_and_expert_hand_example():
    ex = _hand_expert_q2()
    G = oracle.dequant(ex["gate"]["q"], ex["gate"]["scale_bits"], ex["gate"]["min_bits"], 2)
    assert G.tolist() == [[0, 0.5, -2, 1], [-2, 0, 0, -0.5]]
    D = oracle.dequant(ex["down"]["q"], ex["down"]["scale_bits"], ex["down"]["min_bits"], 2)
    assert D.tolist() == [[1, 0], [0, 1], [0.5, 0.5], [0.5, -0.5]]
    x = np.array([1.0, 2.0, 0.5, -1.0])
    # g = [-1, -1.5]; u = [1, -2]; h = silu(g) * u
    h0 = -1.0 / (1 + math.exp(1.0))
    h1 = -1.5 / (1 + math.exp(1.5)) * -2.0
    y = oracle.expert_ffn(ex, x, 2)
    assert np.allclose(y, [h0, h1, 0.5 * (h0 + h1), 0.5 * (h0 - h1)], rtol=1e-15, atol=1e-17)


def test_q2_dequant_mid_code_zero_round_trip_and_float32_exact():
    dims = synth.Dims(128, 64, 4, 2, 64, bits=2)
    for mat in (synth.MAT_UP, synth.MAT_DOWN):
        q = synth.expert_codes(1337, dims, 0, 2, mat)
        assert q.max() <= 3 and set(np.unique(q).tolist()) == {0, 1, 2, 3}
        sb, mb = synth.expert_params_bits(1337, dims, 0, 2, mat)
        W = oracle.dequant(q, sb, mb, dims.chunk)
        s = np.repeat(oracle.bf16_to_f64(sb), dims.chunk, 1)
        m = np.repeat(oracle.bf16_to_f64(mb), dims.chunk, 1)
        assert np.all(W[q == 2] == 0.0)                         # min = -2 * scale
        assert np.array_equal(np.rint((W - m) / s).astype(np.uint8), q)
        w32 = (s.astype(np.float32) * q.astype(np.float32)) + m.astype(np.float32)
        assert np.array_equal(w32.astype(np.float64), W)


def test_q2_quantisation_error_bound():
    # A 4-level affine grid spanning each chunk: dequant(quant(v)) is within
    # half a step of v.
    rng = np.random.default_rng(13)
    v = rng.uniform(-0.05, 0.05, (8, 64))
    sb = synth.bf16_bits_from_f64((v.max(1) - v.min(1)) / 3.0)[:, None]
    mb = synth.bf16_bits_from_f64(v.min(1))[:, None]
    sv, mv = oracle.bf16_to_f64(sb), oracle.bf16_to_f64(mb)
    q = np.clip(np.rint((v - mv) / sv), 0, 3).astype(np.uint8)
    W = oracle.dequant(q, sb, mb, 64)
    inside = (v >= mv) & (v <= mv + 3 * sv)
    bound = np.broadcast_to(sv / 2 + 1e-15, v.shape)
    assert np.all(np.abs(W - v)[inside] <= bound[inside])


def test_q2_single_expert_weight_one_is_dense_swiglu():
    dims = synth.Dims(256, 128, 16, 1, 64, bits=2)
    dims, experts, wr = _tiny_stack(dims=dims)
    r = synth.hidden_bf16(1337, 1, dims.d_model).astype(np.float64)
    out = oracle.moe_layer(r, wr, experts, dims)
    assert out["w"].tolist() == [1.0]
    dense = _dense_swiglu_torch(experts[out["idx"][0]], out["x"], dims.chunk)
    assert np.allclose(out["y"], dense, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# Prefill union
# ---------------------------------------------------------------------------
def _random_idx(rng, T, E, k):
    return [list(rng.choice(E, k, replace=False)) for _ in range(T)]


def test_union_properties_and_independent_order():
    rng = np.random.default_rng(13)
    for T, E, k in ((64, 128, 8), (17, 16, 4), (1, 128, 8), (64, 16, 4), (3, 8, 8)):
        idx = _random_idx(rng, T, E, k)
        U, counts, offsets, perm = oracle.expert_union(idx)
        flat = np.array(idx).reshape(-1)
        assert sorted(U) == sorted(set(flat.tolist()))
        assert len(U) <= min(E, T * k)
        assert sum(counts) == T * k and offsets[-1] == T * k
        assert sorted(perm) == list(range(T * k))
        # independent first-touch order: numpy unique with first positions
        uniq, first = np.unique(flat, return_index=True)
        assert U == [int(u) for u in uniq[np.argsort(first)]]
        for u, e in enumerate(U):
            seg = perm[offsets[u]:offsets[u + 1]]
            assert all(flat[p] == e for p in seg)
            ts = [p // k for p in seg]
            assert ts == sorted(ts)
            assert counts[u] == int(np.sum(flat == e))


def test_union_single_token_is_its_routing():
    U, counts, offsets, perm = oracle.expert_union([[5, 2, 9, 0]])
    assert U == [5, 2, 9, 0] and counts == [1, 1, 1, 1] and perm == [0, 1, 2, 3]


def test_prefill_chunk_equals_per_token_decode():
    dims, experts, wr = _tiny_stack()
    rs = [synth.hidden_bf16(1337, 100 + t, dims.d_model).astype(np.float64) for t in range(5)]
    pc = oracle.prefill_chunk(rs, wr, experts, dims)
    for t, r in enumerate(rs):
        d = oracle.moe_layer(r, wr, experts, dims)
        assert d["idx"] == pc["tokens"][t]["idx"]
        assert np.array_equal(d["y"], pc["tokens"][t]["y"])


# ---------------------------------------------------------------------------
# LRU ring
# ---------------------------------------------------------------------------
class _LruOrderedDict:
    """An independent LRU model: OrderedDict in recency order, pins as a set,
    empty slots handed out in index order."""

    def __init__(self, n):
        self.n = n
        self.od = OrderedDict()     # key -> slot, least recent first
        self.next_empty = 0
        self.pins = set()

    def layer(self, L, experts):
        self.pins = set()
        out = []
        for r, e in enumerate(experts):
            key = (L, int(e))
            if key in self.od:
                self.od.move_to_end(key)
                out.append((L, r, int(e), 0, self.od[key], None))
            else:
                if self.next_empty < self.n:
                    s, ev = self.next_empty, None
                    self.next_empty += 1
                else:
                    ev = next(k for k in self.od if k not in self.pins)
                    s = self.od.pop(ev)
                self.od[key] = s
                out.append((L, r, int(e), 1, s, ev))
            self.pins.add(key)
        return out

    def prefetch(self, L, experts):
        out = []
        for r, e in enumerate(experts):
            key = (L, int(e))
            if key in self.od:
                continue
            if self.next_empty < self.n:
                s, ev = self.next_empty, None
                self.next_empty += 1
            else:
                ev = next((k for k in self.od if k not in self.pins), None)
                if ev is None:
                    break
                s = self.od.pop(ev)
            self.od[key] = s
            out.append((L, r, int(e), 2, s, ev))
        return out


def _routing_trace(rng, T, L, E, k, reuse=0.5):
    trace, prev = [], None
    for t in range(T):
        layers = []
        for l in range(L):
            if prev is not None and rng.random() < reuse:
                base = list(prev[l])
                rng.shuffle(base)
                keep = base[: k // 2]
                rest = [e for e in rng.permutation(E) if e not in keep][: k - len(keep)]
                sel = keep + list(rest)
            else:
                sel = list(rng.choice(E, k, replace=False))
            layers.append([int(e) for e in sel])
        trace.append(layers)
        prev = layers
    return trace


@pytest.mark.parametrize("n_slots", [4, 8, 13, 40, 500])
def test_lru_two_independent_simulators_agree(n_slots):
    rng = np.random.default_rng(14 + n_slots)
    T, L, E, k = 12, 5, 16, 4
    trace = _routing_trace(rng, T, L, E, k)
    events, (h, m, ev) = oracle.ring_trace(trace, n_slots)
    ref = _LruOrderedDict(n_slots)
    ref_events = []
    for t, layers in enumerate(trace):
        for l, experts in enumerate(layers):
            ref_events.extend((t,) + e for e in ref.layer(l, experts))
    assert events == ref_events
    assert h + m == T * L * k


def test_lru_large_ring_only_cold_misses():
    rng = np.random.default_rng(15)
    T, L, E, k = 10, 4, 16, 4
    trace = _routing_trace(rng, T, L, E, k)
    events, (h, m, ev) = oracle.ring_trace(trace, L * E)
    distinct = {(l, e) for layers in trace for l, exps in enumerate(layers) for e in exps}
    assert m == len(distinct) and ev == 0


def test_lru_ring_of_k_slots_misses_every_new_layer():
    rng = np.random.default_rng(16)
    T, L, E, k = 4, 3, 16, 4
    trace = _routing_trace(rng, T, L, E, k)
    events, (h, m, ev) = oracle.ring_trace(trace, k)
    assert h == 0 and m == T * L * k


def test_lru_repeated_token_all_hits():
    rng = np.random.default_rng(17)
    L, E, k = 6, 16, 4
    tok = [[int(e) for e in rng.choice(E, k, replace=False)] for _ in range(L)]
    events, (h, m, ev) = oracle.ring_trace([tok, tok, tok], L * k)
    assert m == L * k and h == 2 * L * k


def test_lru_never_evicts_current_layer():
    rng = np.random.default_rng(18)
    T, L, E, k = 20, 3, 16, 4
    trace = _routing_trace(rng, T, L, E, k, reuse=0.8)
    events, _ = oracle.ring_trace(trace, k + 1)
    for (t, l, r, e, kind, s, evicted) in events:
        if evicted is not None:
            assert evicted[0] != l or evicted[1] not in trace[t][l][:r]


@pytest.mark.parametrize("n_slots", [4, 9, 30, 200])
def test_lru_prefetch_two_independent_simulators_agree(n_slots):
    """Speculative loads after every layer (ranks past k, drawn at random):
    the oracle's prefetch and an OrderedDict model give the same events."""
    rng = np.random.default_rng(40 + n_slots)
    T, L, E, k, N = 10, 4, 16, 4, 5
    trace = _routing_trace(rng, T, L, E, k)
    a, b = oracle.LruRing(n_slots), _LruOrderedDict(n_slots)
    ev_a, ev_b = [], []
    for layers in trace:
        for l, experts in enumerate(layers):
            a.release()
            ev_a.extend(a.acquire(l, experts))
            ev_b.extend(b.layer(l, experts))
            bets = [int(e) for e in rng.permutation(E) if e not in experts][:N]
            ev_a.extend(a.prefetch(l, bets))
            ev_b.extend(b.prefetch(l, bets))
    assert ev_a == ev_b
    assert a.prefetches == sum(1 for e in ev_a if e[3] == oracle.PREFETCH)


def test_prefetch_then_request_is_a_hit_and_a_resident_bet_is_free():
    ring = oracle.LruRing(8)
    ring.acquire(0, [1, 2])
    ev = ring.prefetch(0, [3, 1, 4])              # 1 is resident: no event, no tick
    assert [(e[2], e[3], e[4]) for e in ev] == [(3, oracle.PREFETCH, 2), (4, oracle.PREFETCH, 3)]
    ring.release()
    got = ring.acquire(1, [3])                     # another layer's expert 3: a miss
    assert got[0][3] == oracle.MISS
    ring.release()
    got = ring.acquire(0, [3, 4])                  # the bets pay off
    assert [e[3] for e in got] == [oracle.HIT, oracle.HIT]
    assert ring.hits == 2 and ring.misses == 3 and ring.prefetches == 2


def test_prefetch_never_displaces_the_current_acquisition():
    ring = oracle.LruRing(4)
    ring.acquire(0, [0, 1, 2, 3])                  # every slot pinned
    assert ring.prefetch(0, [4, 5]) == []
    ring.release()
    ev = ring.prefetch(0, [4])                     # now the oldest slot goes
    assert ev == [(0, 0, 4, oracle.PREFETCH, 0, (0, 0))]


def test_prefetch_evicts_in_lru_order_after_bets():
    # a bet gets a fresh tick, so older demand entries go first
    ring = oracle.LruRing(3)
    ring.acquire(0, [0])
    ring.release()
    ring.acquire(1, [0])
    ring.release()
    ring.prefetch(2, [0])                          # fills the last empty slot
    ev = ring.prefetch(3, [0])                     # evicts (0, 0), the oldest
    assert ev[0][5] == (0, 0)
