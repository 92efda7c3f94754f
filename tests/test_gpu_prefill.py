"""GPU parity of layer-major prefill (expert union, permutation, grouped MFMA
expert FFN, combine) against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import quantised_routed_expert_amd as smoe
import synth
from synth.device import DeviceStack
from tests.gpu_common import (LazyExperts, check_moe_output, check_prefill_against_oracle, need_gpu,
                              random_residual, say)

pytestmark = pytest.mark.gpu

SHAPES = {
    "tiny": synth.Dims(256, 128, 16, 4, 32),
    "ragged": synth.Dims(768, 384, 24, 3, 64),
    "q235b": synth.Dims(4096, 1536, 128, 8, 64),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    torch.cuda.init()


def run_prefill(dims, stack, layer, res_np):
    """route + prefill_chunk on the GPU for a [T][d] chunk."""
    T = res_np.shape[0]
    r = torch.from_numpy(res_np.copy()).cuda()
    x = torch.empty((T, dims.d_model), dtype=torch.int16, device="cuda")
    idx = torch.empty((T, dims.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, dims.top_k), dtype=torch.float32, device="cuda")
    mu = min(dims.n_experts, T * dims.top_k)
    uids = torch.full((mu,), -7, dtype=torch.int32, device="cuda")
    ucount = torch.zeros(1, dtype=torch.int32, device="cuda")
    offs = torch.full((mu + 1,), -7, dtype=torch.int32, device="cuda")
    perm = torch.full((T * dims.top_k,), -7, dtype=torch.int32, device="cuda")
    ws = smoe.workspace(dims, T)
    smoe.route(dims, r, x, stack.router_layer(layer), stack.bias_layer(layer), idx, w, ws)
    smoe.moe_prefill_chunk(dims, x, idx, w, stack.table(layer), r, uids, ucount, offs, perm, ws)
    torch.cuda.synchronize()
    n = int(ucount.item())
    return {"idx": idx.cpu().numpy(), "w": w.cpu().numpy(), "r_out": r.cpu().numpy(),
            "union": uids.cpu().numpy()[:n].tolist(), "offsets": offs.cpu().numpy()[:n + 1].tolist(),
            "perm": perm.cpu().numpy().tolist()}


def check_union(got, T, k):
    U, counts, offsets, perm = oracle.expert_union(got["idx"].tolist())
    assert got["union"] == U
    assert got["offsets"] == offsets
    assert got["perm"] == perm
    return len(U)


@pytest.mark.parametrize("shape,T,zipf", [
    ("tiny", 1, 0.0), ("tiny", 5, 0.0), ("tiny", 64, 0.0),
    ("ragged", 17, 0.0), ("ragged", 64, 1.1),
    ("q235b", 64, 1.1), ("q235b", 9, 0.0),
])
def test_prefill_parity(shape, T, zipf):
    """Every token of the chunk against the oracle (at the 235B shape with the
    Zipf-biased routing: about 70 union experts, many with one or two tokens,
    a few spanning several 16-row slices)."""
    dims = SHAPES[shape]
    say(f"[prefill] {shape} T={T} zipf={zipf}")
    stack = DeviceStack(1337, dims, 1, zipf_s=zipf)
    rng = np.random.default_rng(T)
    res = random_residual(rng, T, dims.d_model, scale=1.5)
    got = run_prefill(dims, stack, 0, res)
    n_union = check_union(got, T, dims.top_k)
    say(f"[prefill] |union| = {n_union}")
    check_prefill_against_oracle(got, res, stack, dims, 0, f"prefill {shape} T={T}")


def test_prefill_all_tokens_same_experts_fills_m_tiles():
    # 64 copies of one hidden state: every union expert has 64 tokens (4 M tiles)
    dims = SHAPES["ragged"]
    stack = DeviceStack(1337, dims, 1)
    h = random_residual(np.random.default_rng(4), 1, dims.d_model)
    res = np.repeat(h, 64, axis=0)
    got = run_prefill(dims, stack, 0, res)
    assert check_union(got, 64, dims.top_k) == dims.top_k
    ref = oracle.moe_layer(h[0].astype(np.float64), stack.router_bits[0], LazyExperts(1337, dims, 0), dims)
    y = got["r_out"].astype(np.float64) - res.astype(np.float64)
    for t in (0, 17, 63):
        check_moe_output(y[t], ref["y"], f"token {t}")
    # identical tokens get bitwise identical outputs
    assert np.all(got["r_out"] == got["r_out"][0:1])


def test_prefill_matches_decode_within_tolerance():
    dims = SHAPES["q235b"]
    stack = DeviceStack(1337, dims, 1)
    res = random_residual(np.random.default_rng(11), 3, dims.d_model)
    got = run_prefill(dims, stack, 0, res)
    ws = smoe.workspace(dims, 1)
    for t in range(3):
        r = torch.from_numpy(res[t:t + 1].copy()).cuda()
        x = torch.empty((1, dims.d_model), dtype=torch.int16, device="cuda")
        idx = torch.empty((1, dims.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((1, dims.top_k), dtype=torch.float32, device="cuda")
        smoe.route(dims, r, x, stack.router_layer(0), None, idx, w, ws)
        smoe.moe_decode(dims, x, idx, w, stack.table(0), r, ws)
        torch.cuda.synchronize()
        yd = r.cpu().numpy()[0].astype(np.float64) - res[t]
        yp = got["r_out"][t].astype(np.float64) - res[t]
        check_moe_output(yp, yd, f"prefill vs decode t{t}")


def test_prefill_is_deterministic():
    dims = SHAPES["q235b"]
    stack = DeviceStack(1337, dims, 1, zipf_s=1.1)
    res = random_residual(np.random.default_rng(12), 64, dims.d_model)
    a = run_prefill(dims, stack, 0, res)
    b = run_prefill(dims, stack, 0, res)
    assert np.array_equal(a["r_out"], b["r_out"])
    assert a["perm"] == b["perm"]


def test_prefill_rejects_bad_token_counts():
    dims = SHAPES["tiny"]
    stack = DeviceStack(1337, dims, 1)
    ws = smoe.workspace(dims, 64)
    x = torch.zeros((65, dims.d_model), dtype=torch.int16, device="cuda")
    idx = torch.zeros((65, dims.top_k), dtype=torch.int32, device="cuda")
    w = torch.zeros((65, dims.top_k), dtype=torch.float32, device="cuda")
    r = torch.zeros((65, dims.d_model), device="cuda")
    z = torch.zeros(1024, dtype=torch.int32, device="cuda")
    with pytest.raises(smoe.SmoeError):
        smoe.moe_prefill_chunk(dims, x, idx, w, stack.table(0), r, z, z, z, z, ws)


def run_prefill_given_routing(dims, stack, table, res_np, idx_np, w_np):
    """smoe_route for x, then smoe_moe_prefill_chunk with the given routing
    (ids and weights) and expert table instead of the router's."""
    T = res_np.shape[0]
    r = torch.from_numpy(res_np.copy()).cuda()
    x = torch.empty((T, dims.d_model), dtype=torch.int16, device="cuda")
    idx = torch.empty((T, dims.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, dims.top_k), dtype=torch.float32, device="cuda")
    ws = smoe.workspace(dims, T)
    smoe.route(dims, r, x, stack.router_layer(0), None, idx, w, ws)
    idx.copy_(torch.from_numpy(np.asarray(idx_np, dtype=np.int32)))
    w.copy_(torch.from_numpy(np.asarray(w_np, dtype=np.float32)))
    mu = min(dims.n_experts, T * dims.top_k)
    uids = torch.full((mu,), -7, dtype=torch.int32, device="cuda")
    ucount = torch.zeros(1, dtype=torch.int32, device="cuda")
    offs = torch.full((mu + 1,), -7, dtype=torch.int32, device="cuda")
    perm = torch.full((T * dims.top_k,), -7, dtype=torch.int32, device="cuda")
    smoe.moe_prefill_chunk(dims, x, idx, w, table, r, uids, ucount, offs, perm, ws)
    torch.cuda.synchronize()
    n = int(ucount.item())
    return {"r_out": r.cpu().numpy(), "union": uids.cpu().numpy()[:n].tolist(),
            "offsets": offs.cpu().numpy()[:n + 1].tolist(), "perm": perm.cpu().numpy().tolist()}


def oracle_mix(res, idx, w, experts, dims, skip=()):
    """y_t = sum_r w[t][r] FFN_{idx[t][r]}(x_t) in rank order (experts in
    ``skip`` contribute nothing), with x_t the oracle's RMSNorm."""
    out = []
    for t in range(res.shape[0]):
        x, _ = oracle.rmsnorm_bf16(res[t].astype(np.float64), dims.rms_eps)
        y = np.zeros(dims.d_model)
        for rk, e in enumerate(idx[t]):
            if int(e) not in skip:
                y = y + float(w[t][rk]) * oracle.expert_ffn(experts[int(e)], x, dims.chunk)
        out.append(y)
    return out


def test_prefill_null_table_entry_contributes_nothing():
    """A routed expert whose table entry is NULL (e.g. a ring table that holds
    only an acquired union) is left out of the union and contributes nothing;
    the other experts' outputs are unchanged."""
    dims = SHAPES["ragged"]
    stack = DeviceStack(1337, dims, 1)
    T = 12
    res = random_residual(np.random.default_rng(31), T, dims.d_model)
    got0 = run_prefill(dims, stack, 0, res)
    idx, w = got0["idx"], got0["w"]
    dropped = int(idx[3][1])
    table = stack.table(0).clone()
    table[dropped] = 0
    got = run_prefill_given_routing(dims, stack, table, res, idx, w)
    U, counts, offsets, perm = oracle.expert_union(idx.tolist())
    keep = [u for u in U if u != dropped]
    assert got["union"] == keep
    ent = [[p for p in perm[offsets[i]:offsets[i + 1]]] for i, u in enumerate(U) if u != dropped]
    assert got["perm"][:sum(len(x) for x in ent)] == [p for x in ent for p in x]
    assert got["offsets"] == list(np.cumsum([0] + [len(x) for x in ent]))
    refs = oracle_mix(res, idx, w, LazyExperts(1337, dims, 0), dims, skip=(dropped,))
    for t in range(T):
        check_moe_output(got["r_out"][t].astype(np.float64) - res[t], refs[t], f"null-entry t{t}")


def test_prefill_repeated_expert_in_a_token():
    """A token that lists one expert twice (the router never does) gets one
    row per entry: the union and permutation equal the oracle's scan, and the
    expert's output counts with both weights."""
    dims = SHAPES["tiny"]
    stack = DeviceStack(1337, dims, 1)
    T, k = 6, dims.top_k
    res = random_residual(np.random.default_rng(32), T, dims.d_model)
    rng = np.random.default_rng(33)
    idx = np.stack([rng.permutation(dims.n_experts)[:k] for _ in range(T)]).astype(np.int32)
    idx[1][2] = idx[1][0]                      # token 1: expert twice
    idx[4][3] = idx[4][1] = idx[4][0]          # token 4: three times
    w = rng.uniform(0.05, 0.5, size=(T, k)).astype(np.float32)
    got = run_prefill_given_routing(dims, stack, stack.table(0), res, idx, w)
    U, counts, offsets, perm = oracle.expert_union(idx.tolist())
    assert got["union"] == U
    assert got["offsets"] == offsets
    assert got["perm"] == perm
    refs = oracle_mix(res, idx, w, LazyExperts(1337, dims, 0), dims)
    for t in range(T):
        check_moe_output(got["r_out"][t].astype(np.float64) - res[t], refs[t], f"repeat t{t}")


def test_prefill_chunks_on_concurrent_streams_match_one_stream():
    """Three 64-token chunks through three chained layers of the 235B shape,
    once one chunk after another on one stream, once as a causal pipeline on
    three streams (chunk c one layer behind chunk c - 1 and waiting for its
    layer, each stream with its own buffers and workspace: the schedule the
    benchmark runs).  The library keeps no state between calls, so the
    residuals must be bitwise equal."""
    dims = SHAPES["q235b"]
    NL, C, n_chunks = 3, 64, 3
    stack = DeviceStack(synth.SEED, dims, NL, zipf_s=1.1)
    say(f"concurrent prefill streams: {n_chunks} chunks x {NL} layers, dims {vars(dims)}")
    prompt = torch.from_numpy(np.stack([synth.hidden_bf16(synth.SEED, 30_000 + t, dims.d_model)
                                        for t in range(C * n_chunks)])).cuda()
    mu = min(dims.n_experts, C * dims.top_k)

    def buffers():
        return dict(x=torch.empty((C, dims.d_model), dtype=torch.int16, device="cuda"),
                    idx=torch.empty((C, dims.top_k), dtype=torch.int32, device="cuda"),
                    w=torch.empty((C, dims.top_k), dtype=torch.float32, device="cuda"),
                    uids=torch.empty(mu, dtype=torch.int32, device="cuda"),
                    uc=torch.zeros(1, dtype=torch.int32, device="cuda"),
                    offs=torch.empty(mu + 1, dtype=torch.int32, device="cuda"),
                    perm=torch.empty(C * dims.top_k, dtype=torch.int32, device="cuda"),
                    ws=smoe.workspace(dims, C))

    def chunk_layer(b, r, L):
        smoe.route(dims, r, b["x"], stack.router_layer(L), stack.bias_layer(L), b["idx"], b["w"], b["ws"])
        smoe.moe_prefill_chunk(dims, b["x"], b["idx"], b["w"], stack.table(L), r, b["uids"], b["uc"], b["offs"],
                               b["perm"], b["ws"])

    seq = prompt.clone()
    b0 = buffers()
    for c in range(n_chunks):
        for L in range(NL):
            chunk_layer(b0, seq[c * C:(c + 1) * C], L)
    torch.cuda.synchronize()

    par = prompt.clone()
    bufs = [buffers() for _ in range(n_chunks)]
    main = torch.cuda.current_stream()
    streams = [main] + [torch.cuda.Stream() for _ in range(n_chunks - 1)]
    done = [[torch.cuda.Event() for _ in range(NL)] for _ in range(n_chunks)]
    for st in streams[1:]:
        st.wait_stream(main)
    for step in range(NL + n_chunks - 1):
        for c in range(n_chunks):
            L = step - c
            if not 0 <= L < NL:
                continue
            with torch.cuda.stream(streams[c]):
                if c > 0:
                    streams[c].wait_event(done[c - 1][L])
                chunk_layer(bufs[c], par[c * C:(c + 1) * C], L)
                done[c][L].record(streams[c])
    for st in streams[1:]:
        main.wait_stream(st)
    torch.cuda.synchronize()
    assert torch.equal(seq, par)
    assert torch.isfinite(seq).all()
