"""GPU parity of the router and the decode expert FFN against the CPU oracle,
through the C ABI (quantised_routed_expert_amd.binding)."""
import numpy as np
import pytest
import torch

import oracle
import quantised_routed_expert_amd as smoe
import synth
from synth.device import DeviceStack, fill_experts, u16_to_device
from tests.gpu_common import (LazyExperts, bits_u16, check_chain_against_oracle, check_moe_output, need_gpu,
                              random_residual, say)

pytestmark = pytest.mark.gpu

SHAPES = {
    "tiny": synth.Dims(256, 128, 16, 4, 32),
    "ragged": synth.Dims(768, 384, 24, 3, 64),
    "q30b": synth.Dims(2048, 768, 128, 8, 64),
    "q235b": synth.Dims(4096, 1536, 128, 8, 64),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    torch.cuda.init()


def test_device_generator_matches_host():
    for name, dims, layer, experts in (("tiny", SHAPES["tiny"], 0, range(16)),
                                      ("q235b", SHAPES["q235b"], 93, (0, 127))):
        say(f"[synth] {name} layer {layer}")
        stride = synth.blob_sections(dims)["stride"]
        buf = torch.empty(len(experts) * stride, dtype=torch.uint8, device="cuda")
        for i, e in enumerate(experts):
            fill_experts(1337, dims, layer, e, 1, buf.data_ptr() + i * stride, stride)
        got = buf.cpu().numpy()
        for i, e in enumerate(experts):
            ref = synth.pack_blob(1337, dims, layer, e)
            assert np.array_equal(got[i * stride:(i + 1) * stride], ref), (name, e)


@pytest.mark.parametrize("shape", ["tiny", "ragged", "q235b"])
@pytest.mark.parametrize("n_tok", [1, 3, 64])
@pytest.mark.parametrize("norm", [True, False])
def test_route_parity(shape, n_tok, norm):
    dims = SHAPES[shape].replace(norm_topk_prob=norm)
    say(f"[route] {shape} n_tok={n_tok} norm={norm}")
    rng = np.random.default_rng(100 + n_tok)
    wr = synth.router_bits(1337, dims, 2)
    bias = synth.zipf_bias(1337, dims, 2) if n_tok == 3 else None
    res = random_residual(rng, n_tok, dims.d_model, scale=3.0)
    d_res = torch.from_numpy(res).cuda()
    x = torch.empty((n_tok, dims.d_model), dtype=torch.int16, device="cuda")
    idx = torch.empty((n_tok, dims.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((n_tok, dims.top_k), dtype=torch.float32, device="cuda")
    ws = smoe.workspace(dims, n_tok)
    smoe.route(dims, d_res, x, u16_to_device(wr), None if bias is None else torch.from_numpy(bias).cuda(),
               idx, w, ws)
    torch.cuda.synchronize()
    xb, ig, wg = bits_u16(x), idx.cpu().numpy(), w.cpu().numpy()
    for t in range(n_tok):
        xv, xbits = oracle.rmsnorm_bf16(res[t].astype(np.float64), dims.rms_eps)
        assert np.array_equal(xb[t], xbits), f"token {t}: x bits differ"
        l = oracle.router_logits(wr, xv, bias)
        ref_idx, ref_w = oracle.select_topk(l, dims.top_k, dims.norm_topk_prob)
        assert list(ig[t]) == ref_idx, f"token {t}"
        assert np.allclose(wg[t], ref_w, rtol=2e-6, atol=1e-7)


def test_route_tie_break_duplicate_rows():
    dims = SHAPES["tiny"]
    wr = synth.router_bits(1337, dims, 0).copy()
    wr[5] = wr[9] = wr[12] = synth.bf16_bits_from_f64(np.full(dims.d_model, 0.03))
    res = np.abs(random_residual(np.random.default_rng(3), 1, dims.d_model))
    d_res = torch.from_numpy(res).cuda()
    x = torch.empty((1, dims.d_model), dtype=torch.int16, device="cuda")
    idx = torch.empty((1, dims.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, dims.top_k), dtype=torch.float32, device="cuda")
    smoe.route(dims, d_res, x, u16_to_device(wr), None, idx, w, smoe.workspace(dims, 1))
    torch.cuda.synchronize()
    got = idx.cpu().numpy()[0].tolist()
    assert got[:3] == [5, 9, 12]
    wv = w.cpu().numpy()[0]
    assert wv[0] == wv[1] == wv[2]
    xv, _ = oracle.rmsnorm_bf16(res[0].astype(np.float64), dims.rms_eps)
    ref_idx, _ = oracle.select_topk(oracle.router_logits(wr, xv), dims.top_k)
    assert got == ref_idx


def _decode_one_layer(dims, stack, layer, res_np, slots=False):
    """route + moe_decode on the GPU for one token; returns x bits, idx, w, r_out."""
    d_res = torch.from_numpy(res_np.reshape(1, -1).copy()).cuda()
    x = torch.empty((1, dims.d_model), dtype=torch.int16, device="cuda")
    idx = torch.empty((1, dims.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, dims.top_k), dtype=torch.float32, device="cuda")
    ws = smoe.workspace(dims, 1)
    smoe.route(dims, d_res, x, stack.router_layer(layer), stack.bias_layer(layer), idx, w, ws)
    if slots:
        torch.cuda.synchronize()
        ptrs = [stack.blob(layer, int(e)).data_ptr() for e in idx.cpu().numpy()[0]]
        smoe.moe_decode_slots(dims, x, w, ptrs, d_res, ws)
    else:
        smoe.moe_decode(dims, x, idx, w, stack.table(layer), d_res, ws)
    torch.cuda.synchronize()
    return bits_u16(x)[0], idx.cpu().numpy()[0], w.cpu().numpy()[0], d_res.cpu().numpy()[0]


@pytest.mark.parametrize("shape,layers,tokens", [("tiny", 1, 4), ("ragged", 2, 3), ("q30b", 2, 2),
                                                 ("q235b", 1, 2)])
def test_decode_layer_parity(shape, layers, tokens):
    dims = SHAPES[shape]
    say(f"[decode] {shape} layers={layers} tokens={tokens}")
    stack = DeviceStack(1337, dims, layers)
    rng = np.random.default_rng(7)
    worst = 0.0
    for L in range(layers):
        experts = LazyExperts(1337, dims, L)
        for t in range(tokens):
            res = random_residual(rng, 1, dims.d_model, scale=2.0)[0]
            xb, ig, wg, r_out = _decode_one_layer(dims, stack, L, res)
            ref = oracle.moe_layer(res.astype(np.float64), stack.router_bits[L], experts, dims)
            assert np.array_equal(xb, ref["x_bits"])
            assert list(ig) == ref["idx"]
            assert np.allclose(wg, ref["w"], rtol=2e-6, atol=1e-7)
            y = r_out.astype(np.float64) - res.astype(np.float64)
            worst = max(worst, check_moe_output(y, ref["y"], f"{shape} L{L} t{t}"))
    say(f"[decode] {shape}: worst rel-L2 {worst:.2e}")


def test_decode_special_routings():
    base = SHAPES["tiny"]
    rng = np.random.default_rng(8)
    for dims in (base.replace(top_k=1), base.replace(top_k=16), base.replace(norm_topk_prob=False),
                 base.replace(chunk=64)):
        say(f"[decode-special] {dims}")
        stack = DeviceStack(1337, dims, 1)
        experts = LazyExperts(1337, dims, 0)
        res = random_residual(rng, 1, dims.d_model)[0]
        xb, ig, wg, r_out = _decode_one_layer(dims, stack, 0, res)
        ref = oracle.moe_layer(res.astype(np.float64), stack.router_bits[0], experts, dims)
        assert list(ig) == ref["idx"]
        check_moe_output(r_out.astype(np.float64) - res, ref["y"], str(dims))


def test_decode_slots_equals_table_path_bitwise():
    dims = SHAPES["q30b"]
    stack = DeviceStack(1337, dims, 1)
    res = random_residual(np.random.default_rng(9), 1, dims.d_model)[0]
    a = _decode_one_layer(dims, stack, 0, res, slots=False)
    b = _decode_one_layer(dims, stack, 0, res, slots=True)
    assert np.array_equal(a[3], b[3])


def run_chain_and_per_layer(dims, stack, h0, n_layers):
    """The chained entry point (with records) and the same token through
    per-layer smoe_route + smoe_moe_decode calls; every record and the final
    residual must be bitwise equal.  Returns (chained output, per-layer
    [(input residual, (x bits, ids, weights, output residual))], id records,
    weight records)."""
    r = torch.from_numpy(h0.copy()).cuda()
    x_rec = torch.empty((n_layers, dims.d_model), dtype=torch.int16, device="cuda")
    i_rec = torch.empty((n_layers, dims.top_k), dtype=torch.int32, device="cuda")
    w_rec = torch.empty((n_layers, dims.top_k), dtype=torch.float32, device="cuda")
    smoe.decode_layers(dims, n_layers, r, stack.router, None, stack.tables, smoe.workspace(dims, 1), x_rec,
                       i_rec, w_rec)
    torch.cuda.synchronize()
    chain = r.cpu().numpy()
    xr, ir, wr = bits_u16(x_rec), i_rec.cpu().numpy(), w_rec.cpu().numpy()
    res = h0.copy()
    per_layer = []
    for L in range(n_layers):
        out = _decode_one_layer(dims, stack, L, res)
        xb, ig, wg, res_next = out
        assert np.array_equal(xb, xr[L]), f"layer {L}: x bits differ from the chained run"
        assert np.array_equal(ig, ir[L]), f"layer {L}: ids differ from the chained run"
        assert np.array_equal(wg, wr[L]), f"layer {L}: weights differ from the chained run"
        per_layer.append((res, out))
        res = res_next
    assert np.array_equal(res, chain), "chained residual differs from the per-layer calls"
    return chain, per_layer, ir, wr


@pytest.mark.parametrize("shape,n_layers,stream", [("q30b", 6, 0), ("q235b", 4, 4)])
def test_decode_layers_chain_matches_per_layer_calls_and_oracle(shape, n_layers, stream):
    """The benchmarked entry point (selection inside gate/up, the router's
    pair-ordered f16 x, the down kernel's router prefetch) at the 30B and 235B
    shapes: bitwise equal to per-layer calls, teacher-forced oracle parity per
    layer, and the free-running oracle chain."""
    dims = SHAPES[shape]
    say(f"[chain] {shape} {n_layers} layers")
    stack = DeviceStack(1337, dims, n_layers)
    h0 = synth.hidden_bf16(1337, stream, dims.d_model)
    chain, per_layer, ir, wr = run_chain_and_per_layer(dims, stack, h0, n_layers)
    check_chain_against_oracle(dims, stack, h0, chain, per_layer, ir, wr, f"chain {shape}")


def test_decode_is_deterministic():
    dims = SHAPES["q235b"]
    stack = DeviceStack(1337, dims, 2)
    h0 = synth.hidden_bf16(1337, 1, dims.d_model)
    outs = []
    for _ in range(3):
        r = torch.from_numpy(h0.copy()).cuda()
        smoe.decode_layers(dims, 2, r, stack.router, None, stack.tables, smoe.workspace(dims, 1))
        torch.cuda.synchronize()
        outs.append(r.cpu().numpy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])


def test_invalid_arguments_are_rejected():
    dims = SHAPES["tiny"]
    ws = smoe.workspace(dims, 1)
    r = torch.zeros((1, dims.d_model), device="cuda")
    x = torch.empty((1, dims.d_model), dtype=torch.int16, device="cuda")
    idx = torch.empty((1, dims.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, dims.top_k), dtype=torch.float32, device="cuda")
    wr = torch.zeros((dims.n_experts, dims.d_model), dtype=torch.int16, device="cuda")
    for bad in (dims.replace(top_k=17), dims.replace(d_model=300), dims.replace(chunk=48),
                dims.replace(top_k=0)):
        with pytest.raises(smoe.SmoeError):
            smoe.route(bad, r, x, wr, None, idx, w, ws)
    with pytest.raises(smoe.SmoeError):
        smoe.route(dims, r, x, wr, None, idx, w, ws[:16])


@pytest.mark.parametrize("case", ["exact_tie", "float_tie", "tie_at_boundary"])
def test_decode_layers_selection_with_ties_matches_oracle(case):
    """The chained entry point selects inside the gate/up kernel with a float
    fast path; ties (exact, or equal only after rounding to float) in the top k
    must take the exact float64 path and agree with the oracle and with
    smoe_route."""
    dims = synth.Dims(256, 128, 128, 8, 32)
    stack = DeviceStack(1337, dims, 1)
    rng = np.random.default_rng({"exact_tie": 21, "float_tie": 22, "tie_at_boundary": 23}[case])
    res = random_residual(rng, 1, dims.d_model)[0]
    j_small = 17
    res[j_small] = 1e-6 * np.abs(res).max()      # an input element too small to move a float logit
    xv, _ = oracle.rmsnorm_bf16(res.astype(np.float64), dims.rms_eps)
    wr = stack.router_bits[0].copy()
    big = synth.bf16_bits_from_f64(0.03 * np.sign(xv) + 0.0)
    if case == "exact_tie":
        for e in (5, 9, 40):
            wr[e] = big                          # three equal logits at the top
    elif case == "float_tie":
        wr[5] = big
        wr[9] = big.copy()
        wr[9][j_small] = np.uint16(int(wr[9][j_small]) + 1)  # one bf16 ulp on a tiny input
    else:
        # seven clear winners and a tie for the last place
        for n, e in enumerate((2, 3, 4, 6, 7, 8, 10)):
            wr[e] = synth.bf16_bits_from_f64((0.05 + 0.001 * n) * np.sign(xv))
        wr[60] = wr[61] = big
    stack.router_bits[0] = wr
    stack.router[0].copy_(u16_to_device(wr))
    lg = oracle.router_logits(wr, xv)
    ref_idx, ref_w = oracle.select_topk(lg, dims.top_k, dims.norm_topk_prob)
    if case == "float_tie":
        assert lg[5] != lg[9] and np.float32(lg[5]) == np.float32(lg[9])
    # chained entry point (selection inside gate/up)
    r = torch.from_numpy(res.copy()).cuda()
    i_rec = torch.empty((1, dims.top_k), dtype=torch.int32, device="cuda")
    w_rec = torch.empty((1, dims.top_k), dtype=torch.float32, device="cuda")
    smoe.decode_layers(dims, 1, r, stack.router, None, stack.tables, smoe.workspace(dims, 1), None, i_rec, w_rec)
    torch.cuda.synchronize()
    got = i_rec.cpu().numpy()[0].tolist()
    assert got == ref_idx, (got, ref_idx)
    assert np.allclose(w_rec.cpu().numpy()[0], ref_w, rtol=2e-6, atol=1e-7)
    # and the separate router agrees bit for bit
    xb, ig, wg, r_out = _decode_one_layer(dims, stack, 0, res)
    assert list(ig) == got and np.array_equal(wg, w_rec.cpu().numpy()[0])
    assert np.array_equal(r_out, r.cpu().numpy())


@pytest.mark.parametrize("E,k", [(256, 8), (16, 16), (24, 3)])
def test_decode_layers_selection_other_expert_counts(E, k):
    """The in-kernel selection has a compile-time path for E <= 128 and a
    general one above; both must agree with the separate router and the oracle."""
    dims = synth.Dims(256, 128, E, k, 32)
    n_layers = 2
    stack = DeviceStack(1337, dims, n_layers)
    h0 = random_residual(np.random.default_rng(E + k), 1, dims.d_model)[0]
    r = torch.from_numpy(h0.copy()).cuda()
    i_rec = torch.empty((n_layers, k), dtype=torch.int32, device="cuda")
    w_rec = torch.empty((n_layers, k), dtype=torch.float32, device="cuda")
    smoe.decode_layers(dims, n_layers, r, stack.router, None, stack.tables, smoe.workspace(dims, 1), None,
                       i_rec, w_rec)
    torch.cuda.synchronize()
    res = h0.copy()
    for L in range(n_layers):
        xb, ig, wg, res_next = _decode_one_layer(dims, stack, L, res)
        ref = oracle.moe_layer(res.astype(np.float64), stack.router_bits[L], LazyExperts(1337, dims, L), dims)
        assert list(ig) == ref["idx"]
        assert np.array_equal(ig, i_rec.cpu().numpy()[L])
        assert np.array_equal(wg, w_rec.cpu().numpy()[L])
        res = res_next
    assert np.array_equal(res, r.cpu().numpy())


def test_decode_layers_non_finite_residual_still_selects_valid_experts():
    """A NaN in the residual makes every logit NaN; the selection ranks NaN as
    -inf, so ties break by index and the experts are 0..k-1 (no invalid id ever
    reaches a blob lookup)."""
    dims = SHAPES["tiny"]
    stack = DeviceStack(1337, dims, 1)
    h0 = random_residual(np.random.default_rng(5), 1, dims.d_model)[0]
    h0[3] = np.nan
    r = torch.from_numpy(h0.copy()).cuda()
    i_rec = torch.empty((1, dims.top_k), dtype=torch.int32, device="cuda")
    smoe.decode_layers(dims, 1, r, stack.router, None, stack.tables, smoe.workspace(dims, 1), None, i_rec, None)
    torch.cuda.synchronize()
    assert i_rec.cpu().numpy()[0].tolist() == list(range(dims.top_k))
    _, ig, _, _ = _decode_one_layer(dims, stack, 0, h0)
    assert list(ig) == list(range(dims.top_k))
