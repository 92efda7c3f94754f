"""The no-allocation decode entry point (smoe_decode_layers_static, for callers
that cannot allocate) against the workspace entry point (smoe_decode_layers),
through the C ABI: bitwise equal results on two calls in a row, the second
smaller than the first, so the library's scratch carries the first call's
contents into the second."""
import numpy as np
import pytest
import torch

import quantised_routed_expert_amd as smoe
import synth
from synth.device import DeviceStack
from tests.gpu_common import bits_u16, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    torch.cuda.init()


def run_both(dims, stack, n_layers, h0):
    outs = []
    for static in (True, False):
        r = torch.from_numpy(h0.copy()).cuda()
        x_rec = torch.empty((n_layers, dims.d_model), dtype=torch.int16, device="cuda")
        i_rec = torch.empty((n_layers, dims.top_k), dtype=torch.int32, device="cuda")
        w_rec = torch.empty((n_layers, dims.top_k), dtype=torch.float32, device="cuda")
        if static:
            smoe.decode_layers_static(dims, n_layers, r, stack.router, None, stack.tables, x_rec, i_rec, w_rec)
        else:
            smoe.decode_layers(dims, n_layers, r, stack.router, None, stack.tables, smoe.workspace(dims, 1), x_rec,
                               i_rec, w_rec)
        torch.cuda.synchronize()
        outs.append((r.cpu().numpy(), bits_u16(x_rec), i_rec.cpu().numpy(), w_rec.cpu().numpy()))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)
    return outs[0]


def test_static_scratch_decode_equals_workspace_decode_twice():
    big = synth.Dims(4096, 1536, 128, 8, 64)              # the 235B decode shape, 3 layers
    small = synth.Dims(2048, 768, 64, 4, 64, bits=2)      # then a smaller SMOE-Q2 stack, 2 layers
    for dims, n_layers, stream in ((big, 3, 7), (small, 2, 8)):
        say(f"[no-alloc] {dims} layers={n_layers}")
        stack = DeviceStack(1337, dims, n_layers)
        h0 = synth.hidden_bf16(1337, stream, dims.d_model)
        out = run_both(dims, stack, n_layers, h0)
        assert np.all(np.isfinite(out[0]))
        del stack
        torch.cuda.empty_cache()


def test_static_scratch_rejects_bad_arguments():
    dims = synth.Dims(256, 128, 16, 4, 32)
    stack = DeviceStack(1337, dims, 1)
    r = torch.zeros(dims.d_model, device="cuda")
    with pytest.raises(smoe.SmoeError):
        smoe.decode_layers_static(dims.replace(top_k=17), 1, r, stack.router, None, stack.tables)
    with pytest.raises(smoe.SmoeError):
        smoe.decode_layers_static(dims, -1, r, stack.router, None, stack.tables)
    smoe.decode_layers_static(dims, 0, None, None, None, None)     # zero layers: a no-op
