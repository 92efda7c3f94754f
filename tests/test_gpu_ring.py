"""The HBM expert ring on the GPU: its hit/miss/eviction log must equal the
oracle's LRU simulation of the same routing trace, and ring-backed decode must
be bitwise equal to decode with every expert resident."""
import numpy as np
import pytest
import torch

import oracle
import quantised_routed_expert_amd as smoe
import synth
from synth.device import DeviceStack
from tests.gpu_common import need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    torch.cuda.init()


def make_ring(dims, stack, n_slots, log_capacity=1 << 20):
    stride = stack.stride
    host = torch.empty(stack.vault.numel(), dtype=torch.uint8, pin_memory=True)
    host.copy_(stack.vault)
    slab = torch.empty(n_slots * stride, dtype=torch.uint8, device="cuda")
    copy_stream = torch.cuda.Stream()
    ring = smoe.Ring(n_slots, stack.n_layers, dims.n_experts, dims.top_k, stack.blob_bytes, stride,
                     host.data_ptr(), stride, slab.data_ptr(), copy_stream, log_capacity)
    return ring, (host, slab, copy_stream)


def ring_decode(dims, stack, ring, hidden):
    """Per token, per layer: route on the GPU, read the experts back, acquire
    them in the ring, run the decode FFN on the slot pointers."""
    ws = smoe.workspace(dims, 1)
    routing, outs = [], []
    x = torch.empty((1, dims.d_model), dtype=torch.int16, device="cuda")
    idx = torch.empty((1, dims.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, dims.top_k), dtype=torch.float32, device="cuda")
    for h in hidden:
        r = torch.from_numpy(h.reshape(1, -1).copy()).cuda()
        layers = []
        for L in range(stack.n_layers):
            smoe.route(dims, r, x, stack.router_layer(L), None, idx, w, ws)
            experts = idx.cpu().numpy()[0].tolist()        # synchronises with the router
            layers.append(experts)
            ptrs = ring.acquire(L, experts)
            smoe.moe_decode_slots(dims, x, w, ptrs, r, ws)
        routing.append(layers)
        outs.append(r.cpu().numpy()[0])
    ring.release()
    return routing, np.stack(outs)


def resident_decode(dims, stack, hidden):
    ws = smoe.workspace(dims, 1)
    outs = []
    for h in hidden:
        r = torch.from_numpy(h.copy()).cuda()
        smoe.decode_layers(dims, stack.n_layers, r, stack.router, None, stack.tables, ws)
        outs.append(r.cpu().numpy())
    return np.stack(outs)


@pytest.mark.parametrize("n_slots", [64, 96, 200])
def test_ring_log_matches_oracle_lru_and_output_matches_resident(n_slots):
    dims = synth.Dims(256, 128, 128, 8, 32)
    n_layers, n_tok = 6, 12
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
    assert h + m == n_tok * n_layers * dims.top_k
    assert stats["h2d_bytes"] == m * stack.blob_bytes
    say(f"[ring] slots={n_slots}: hits {h} misses {m} evictions {ev}")
    assert np.array_equal(got, resident_decode(dims, stack, hidden))


def test_ring_repeated_token_hits_and_reuse_across_tokens():
    dims = synth.Dims(256, 128, 16, 4, 32)
    n_layers = 4                       # 64 keys fit a 64-slot ring: only cold misses
    stack = DeviceStack(1337, dims, n_layers)
    h = synth.markov_hidden(1337, 1, dims.d_model)
    ring, keep = make_ring(dims, stack, 64)
    routing, got = ring_decode(dims, stack, ring, np.repeat(h, 3, axis=0))
    stats = ring.stats()
    ring.destroy()
    assert stats["misses"] == n_layers * dims.top_k and stats["hits"] == 2 * n_layers * dims.top_k
    assert np.array_equal(got[0], got[1]) and np.array_equal(got[1], got[2])


def test_ring_argument_errors():
    dims = synth.Dims(256, 128, 16, 4, 32)
    stack = DeviceStack(1337, dims, 2)
    with pytest.raises(smoe.SmoeError):
        make_ring(dims, stack, 63)     # below the [64, 4096] clamp
    with pytest.raises(smoe.SmoeError):
        make_ring(dims, stack, 4097)
    ring, keep = make_ring(dims, stack, 64)
    with pytest.raises(smoe.SmoeError):
        ring.acquire(0, [1, 1, 2, 3])  # duplicate expert
    with pytest.raises(smoe.SmoeError):
        ring.acquire(2, [0, 1, 2, 3])  # layer out of range
    with pytest.raises(smoe.SmoeError):
        ring.acquire(0, [0, 1, 2, 16])  # expert out of range
    ring.acquire(0, [0, 1, 2, 3])
    with pytest.raises(smoe.SmoeError) as e:
        ring.destroy()                 # slots still held
    assert e.value.code == -4
    ring.release()
    torch.cuda.synchronize()
    ring.destroy()
