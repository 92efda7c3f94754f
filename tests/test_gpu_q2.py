"""SMOE-Q2 on the GPU (the 2-bit vault of the Optimizations page, "Q2 Vaults
-- the Next 2x, Twice Over"): the device generator, per-layer and chained
decode and layer-major prefill against the CPU oracle, ring-backed decode
against resident decode and the oracle's LRU run, and the argument checks,
all through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import quantised_routed_expert_amd as smoe
import synth
from synth.device import DeviceStack, fill_experts
from tests.gpu_common import (LazyExperts, check_chain_against_oracle, check_moe_output, check_prefill_against_oracle,
                              need_gpu, random_residual, say)
from tests.test_gpu_decode import _decode_one_layer, run_chain_and_per_layer
from tests.test_gpu_prefill import check_union, run_prefill
from tests.test_gpu_ring import make_ring, resident_decode, ring_decode

pytestmark = pytest.mark.gpu

Q2 = {
    "small": synth.Dims(512, 256, 16, 4, 64, bits=2),
    "ragged": synth.Dims(1536, 384, 24, 3, 64, bits=2),
    "q30b": synth.Dims(2048, 768, 128, 8, 64, bits=2),
    "q235b": synth.Dims(4096, 1536, 128, 8, 64, bits=2),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    torch.cuda.init()


def test_q2_device_generator_matches_host():
    for name, dims, layer, experts in (("small", Q2["small"], 0, range(16)),
                                      ("q235b", Q2["q235b"], 93, (0, 127))):
        say(f"[q2-synth] {name} layer {layer}")
        stride = synth.blob_sections(dims)["stride"]
        buf = torch.empty(len(experts) * stride, dtype=torch.uint8, device="cuda")
        for i, e in enumerate(experts):
            fill_experts(1337, dims, layer, e, 1, buf.data_ptr() + i * stride, stride)
        got = buf.cpu().numpy()
        for i, e in enumerate(experts):
            assert np.array_equal(got[i * stride:(i + 1) * stride], synth.pack_blob(1337, dims, layer, e)), (name, e)


@pytest.mark.parametrize("shape,layers,tokens", [("small", 1, 4), ("ragged", 2, 3), ("q30b", 2, 2),
                                                 ("q235b", 1, 2)])
def test_q2_decode_layer_parity(shape, layers, tokens):
    dims = Q2[shape]
    say(f"[q2-decode] {shape} layers={layers} tokens={tokens}")
    stack = DeviceStack(1337, dims, layers)
    rng = np.random.default_rng(17)
    worst = 0.0
    for L in range(layers):
        experts = LazyExperts(1337, dims, L)
        for t in range(tokens):
            res = random_residual(rng, 1, dims.d_model, scale=2.0)[0]
            xb, ig, wg, r_out = _decode_one_layer(dims, stack, L, res, slots=(t % 2 == 1))
            ref = oracle.moe_layer(res.astype(np.float64), stack.router_bits[L], experts, dims)
            assert np.array_equal(xb, ref["x_bits"])
            assert list(ig) == ref["idx"]
            assert np.allclose(wg, ref["w"], rtol=2e-6, atol=1e-7)
            y = r_out.astype(np.float64) - res.astype(np.float64)
            worst = max(worst, check_moe_output(y, ref["y"], f"q2 {shape} L{L} t{t}"))
    say(f"[q2-decode] {shape}: worst rel-L2 {worst:.2e}")


def test_q2_special_routings_and_size_bounds():
    base = Q2["small"]
    rng = np.random.default_rng(18)
    for dims in (base.replace(top_k=1), base.replace(top_k=16), base.replace(norm_topk_prob=False),
                 base.replace(d_model=8192, d_ff=128), base.replace(d_ff=8192)):
        say(f"[q2-special] {dims}")
        stack = DeviceStack(1337, dims, 1)
        experts = LazyExperts(1337, dims, 0)
        res = random_residual(rng, 1, dims.d_model)[0]
        xb, ig, wg, r_out = _decode_one_layer(dims, stack, 0, res)
        ref = oracle.moe_layer(res.astype(np.float64), stack.router_bits[0], experts, dims)
        assert list(ig) == ref["idx"]
        check_moe_output(r_out.astype(np.float64) - res, ref["y"], str(dims))


@pytest.mark.parametrize("shape,n_layers,stream", [("q30b", 5, 2), ("q235b", 4, 5)])
def test_q2_decode_layers_chain_matches_per_layer_calls_and_oracle(shape, n_layers, stream):
    """The chained SMOE-Q2 entry point at the 30B and 235B shapes: bitwise
    equal to per-layer calls, teacher-forced oracle parity per layer, and the
    free-running oracle chain."""
    dims = Q2[shape]
    say(f"[q2-chain] {shape} {n_layers} layers")
    stack = DeviceStack(1337, dims, n_layers)
    h0 = synth.hidden_bf16(1337, stream, dims.d_model)
    chain, per_layer, ir, wr = run_chain_and_per_layer(dims, stack, h0, n_layers)
    check_chain_against_oracle(dims, stack, h0, chain, per_layer, ir, wr, f"q2 chain {shape}")


def test_q2_decode_is_deterministic():
    dims = Q2["q235b"]
    stack = DeviceStack(1337, dims, 2)
    h0 = synth.hidden_bf16(1337, 3, dims.d_model)
    outs = []
    for _ in range(3):
        r = torch.from_numpy(h0.copy()).cuda()
        smoe.decode_layers(dims, 2, r, stack.router, None, stack.tables, smoe.workspace(dims, 1))
        torch.cuda.synchronize()
        outs.append(r.cpu().numpy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])


@pytest.mark.parametrize("n_slots", [64, 120])
def test_q2_ring_log_matches_oracle_lru_and_output_matches_resident(n_slots):
    dims = synth.Dims(512, 128, 128, 8, 64, bits=2)
    n_layers, n_tok = 5, 10
    stack = DeviceStack(1337, dims, n_layers)
    hidden = synth.markov_hidden(1337, n_tok, dims.d_model)
    ring, keep = make_ring(dims, stack, n_slots)
    routing, got = ring_decode(dims, stack, ring, hidden)
    log = ring.log(1 << 20)
    stats = ring.stats()
    ring.destroy()
    ref_events, (h, m, ev) = oracle.ring_trace(routing, n_slots)
    assert [e[1:] for e in ref_events] == log
    assert (stats["hits"], stats["misses"], stats["evictions"]) == (h, m, ev)
    assert stats["h2d_bytes"] == m * stack.blob_bytes == m * synth.blob_sections(dims)["bytes"]
    say(f"[q2-ring] slots={n_slots}: hits {h} misses {m} evictions {ev}")
    assert np.array_equal(got, resident_decode(dims, stack, hidden))


def test_q2_argument_checks():
    dims = Q2["small"]
    ws = smoe.workspace(dims, 4)
    x = torch.zeros((4, dims.d_model), dtype=torch.int16, device="cuda")
    idx = torch.zeros((4, dims.top_k), dtype=torch.int32, device="cuda")
    w = torch.zeros((4, dims.top_k), dtype=torch.float32, device="cuda")
    table = torch.zeros(dims.n_experts, dtype=torch.int64, device="cuda")
    r = torch.zeros((4, dims.d_model), dtype=torch.float32, device="cuda")
    u = torch.zeros(dims.n_experts + 1, dtype=torch.int32, device="cuda")
    for bad in (dims.replace(chunk=32), synth.Dims(256, 128, 16, 4, 64, bits=2)):
        with pytest.raises(smoe.SmoeError, match="Q2"):
            smoe.moe_decode(bad, x[0], idx[0], w[0], table, r[0], ws)


@pytest.mark.parametrize("E,k", [(256, 8), (24, 3)])
def test_q2_decode_layers_selection_other_expert_counts(E, k):
    """The in-kernel top-k of the chained entry point (general path above 128
    experts) on SMOE-Q2 blobs: equal to the per-layer calls and the oracle."""
    dims = synth.Dims(512, 128, E, k, 64, bits=2)
    n_layers = 2
    stack = DeviceStack(1337, dims, n_layers)
    h0 = random_residual(np.random.default_rng(E + k + 2), 1, dims.d_model)[0]
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
        check_moe_output(res_next.astype(np.float64) - res.astype(np.float64), ref["y"], f"q2 E{E} k{k} L{L}")
        res = res_next
    assert np.array_equal(res, r.cpu().numpy())


# d_ff 256, 384, 768 and 1536 take the down GEMM's K blocks of 256, 128, 256
# and 512 codes (8-byte code loads at 128)
@pytest.mark.parametrize("shape,T,zipf", [
    ("small", 1, 0.0), ("small", 64, 0.0), ("ragged", 17, 1.1), ("ragged", 64, 0.0),
    ("q30b", 64, 1.1), ("q235b", 64, 1.1), ("q235b", 9, 0.0),
])
def test_q2_prefill_parity(shape, T, zipf):
    dims = Q2[shape]
    say(f"[q2-prefill] {shape} T={T} zipf={zipf}")
    stack = DeviceStack(1337, dims, 1, zipf_s=zipf)
    res = random_residual(np.random.default_rng(T + 3), T, dims.d_model, scale=1.5)
    got = run_prefill(dims, stack, 0, res)
    say(f"[q2-prefill] |union| = {check_union(got, T, dims.top_k)}")
    check_prefill_against_oracle(got, res, stack, dims, 0, f"q2 prefill {shape} T={T}")


@pytest.mark.parametrize("dims,T", [
    # the largest K of the folded gate/up GEMM (16 blocks of 512) and a d_ff of one down block
    (synth.Dims(8192, 512, 32, 4, 64, bits=2), 17),
    # 256 experts, top-16: up to 256 union experts and their slices; d_ff 8192 (16 down blocks)
    (synth.Dims(512, 256, 256, 16, 64, bits=2), 64),
    (synth.Dims(512, 8192, 16, 4, 64, bits=2), 33),
], ids=["d_model_8192", "e256_k16", "d_ff_8192"])
def test_q2_prefill_size_bounds(dims, T):
    say(f"[q2-prefill-bound] {dims} T={T}")
    stack = DeviceStack(1337, dims, 1)
    res = random_residual(np.random.default_rng(T + 5), T, dims.d_model, scale=1.5)
    got = run_prefill(dims, stack, 0, res)
    say(f"[q2-prefill-bound] |union| = {check_union(got, T, dims.top_k)}")
    check_prefill_against_oracle(got, res, stack, dims, 0, f"q2 bound T={T}")


def test_q2_prefill_full_m_tiles_and_matches_decode():
    """64 copies of one hidden state (every union expert gets 4 M tiles of 16
    rows): bitwise equal rows, and within tolerance of SMOE-Q2 decode."""
    dims = Q2["q30b"]
    stack = DeviceStack(1337, dims, 1)
    h = random_residual(np.random.default_rng(21), 1, dims.d_model)
    res = np.repeat(h, 64, axis=0)
    got = run_prefill(dims, stack, 0, res)
    assert check_union(got, 64, dims.top_k) == dims.top_k
    assert np.all(got["r_out"] == got["r_out"][0:1])
    _, _, _, r_dec = _decode_one_layer(dims, stack, 0, h[0])
    check_moe_output(got["r_out"][0].astype(np.float64) - h[0], r_dec.astype(np.float64) - h[0],
                     "q2 prefill vs decode")
