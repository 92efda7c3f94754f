"""Magnitude edge cases of the expert FFN on the GPU: per-chunk scales drawn
from U(0.05, 0.1) (five to fifty times the synthetic stack's), a residual with
outlier channels, and in every expert a few gate/up rows whose codes follow
the sign of the input, so that |silu(g) * u| reaches 10^5 .. 10^7 -- beyond
the largest fp16 value (65504).  Decode and layer-major prefill, SMOE-Q4 and
SMOE-Q2, against the oracle at the usual tolerance."""
import numpy as np
import pytest
import torch

import oracle
import quantised_routed_expert_amd as smoe
import synth
from synth.device import DeviceStack
from tests.gpu_common import check_moe_output, need_gpu, say
from tests.test_gpu_decode import _decode_one_layer
from tests.test_gpu_prefill import check_union, run_prefill

pytestmark = pytest.mark.gpu

F16_MAX = 65504.0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    torch.cuda.init()


def big_expert(rng, dims, direction, planted):
    """Codes uniform over the code range, per-chunk scale ~U(0.05, 0.1) in
    bf16, min = -(mid code) * scale; the gate and up rows in ``planted`` take
    the top code where ``direction`` is positive and code 0 elsewhere."""
    top = (1 << dims.bits) - 1
    mid = float(1 << (dims.bits - 1))
    out = {}
    for name, rows, cols in (("gate", dims.d_ff, dims.d_model), ("up", dims.d_ff, dims.d_model),
                             ("down", dims.d_model, dims.d_ff)):
        q = rng.integers(0, top + 1, size=(rows, cols), dtype=np.uint8)
        if name != "down":
            q[planted] = np.where(direction > 0, top, 0).astype(np.uint8)
        s = synth.bf16_bits_from_f64(rng.uniform(0.05, 0.1, size=(rows, cols // dims.chunk)))
        m = synth.bf16_bits_from_f64(-mid * synth.bf16_bits_to_f64(s))
        out[name] = {"q": q, "scale_bits": s, "min_bits": m}
    return out


def big_stack(dims, seed):
    rng = np.random.default_rng(seed)
    direction = rng.standard_normal(dims.d_model)
    stack = DeviceStack(1337, dims, 1)
    experts = {}
    for e in range(dims.n_experts):
        planted = rng.choice(dims.d_ff, size=8, replace=False)
        experts[e] = big_expert(rng, dims, direction, planted)
        stack.blob(0, e).copy_(torch.from_numpy(synth.pack_logical(dims, experts[e])))
    torch.cuda.synchronize()
    return stack, experts, direction, rng


def big_residual(rng, direction, n_tok):
    d = direction.size
    r = 2.0 * direction[None, :] + 0.5 * rng.standard_normal((n_tok, d))
    r[:, :4] += 20.0                       # outlier channels
    return r.astype(np.float32)


SHAPES = {"q4": synth.Dims(4096, 512, 16, 4, 64), "q2": synth.Dims(4096, 512, 16, 4, 64, bits=2)}


@pytest.mark.parametrize("fmt", ["q4", "q2"])
def test_decode_activations_beyond_fp16_range(fmt):
    dims = SHAPES[fmt]
    stack, experts, direction, rng = big_stack(dims, 31)
    res = big_residual(rng, direction, 3)
    for t in range(3):
        ref = oracle.moe_layer(res[t].astype(np.float64), stack.router_bits[0], experts, dims, return_h=True)
        hmax = max(np.max(np.abs(h)) for h in ref["h"])
        say(f"[range] decode {fmt} t{t}: max |h| {hmax:.3e}")
        assert hmax > F16_MAX, "the case must exceed the fp16 range"
        xb, ig, wg, r_out = _decode_one_layer(dims, stack, 0, res[t])
        assert list(ig) == ref["idx"]
        check_moe_output(r_out.astype(np.float64) - res[t].astype(np.float64), ref["y"], f"{fmt} decode t{t}")


@pytest.mark.parametrize("fmt", ["q4", "q2"])
def test_prefill_activations_beyond_fp16_range(fmt):
    dims = SHAPES[fmt]
    stack, experts, direction, rng = big_stack(dims, 32)
    T = 40
    res = big_residual(rng, direction, T)
    got = run_prefill(dims, stack, 0, res)
    check_union(got, T, dims.top_k)
    for t in range(T):
        ref = oracle.moe_layer(res[t].astype(np.float64), stack.router_bits[0], experts, dims)
        assert got["idx"][t].tolist() == ref["idx"], f"token {t}"
        y = got["r_out"][t].astype(np.float64) - res[t].astype(np.float64)
        check_moe_output(y, ref["y"], f"{fmt} prefill t{t}")
