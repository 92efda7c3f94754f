"""GPU parity of layer-major prefill (expert union, permutation, grouped MFMA
expert FFN, combine) against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import quantised_routed_expert_amd as smoe
import synth
from synth.device import DeviceStack
from tests.gpu_common import LazyExperts, check_moe_output, need_gpu, random_residual, say

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


@pytest.mark.parametrize("shape,T,zipf,sample", [
    ("tiny", 1, 0.0, None), ("tiny", 5, 0.0, None), ("tiny", 64, 0.0, None),
    ("ragged", 17, 0.0, None), ("ragged", 64, 1.1, None),
    ("q235b", 64, 1.1, [0, 13, 40, 63]), ("q235b", 9, 0.0, [0, 8]),
])
def test_prefill_parity(shape, T, zipf, sample):
    dims = SHAPES[shape]
    say(f"[prefill] {shape} T={T} zipf={zipf}")
    stack = DeviceStack(1337, dims, 1, zipf_s=zipf)
    rng = np.random.default_rng(T)
    res = random_residual(rng, T, dims.d_model, scale=1.5)
    got = run_prefill(dims, stack, 0, res)
    n_union = check_union(got, T, dims.top_k)
    say(f"[prefill] |union| = {n_union}")
    experts = LazyExperts(1337, dims, 0)
    toks = range(T) if sample is None else sample
    worst = 0.0
    for t in toks:
        ref = oracle.moe_layer(res[t].astype(np.float64), stack.router_bits[0], experts, dims,
                               bias=None if stack.bias_np is None else stack.bias_np[0])
        assert got["idx"][t].tolist() == ref["idx"], f"token {t}"
        assert np.allclose(got["w"][t], ref["w"], rtol=2e-6, atol=1e-7)
        y = got["r_out"][t].astype(np.float64) - res[t].astype(np.float64)
        worst = max(worst, check_moe_output(y, ref["y"], f"{shape} t{t}"))
    say(f"[prefill] {shape} T={T}: worst rel-L2 {worst:.2e}")


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
