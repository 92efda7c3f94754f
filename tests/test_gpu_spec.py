"""Speculative ring loads on the GPU, through the C ABI: the router's ranking
past the top k (the bets), ring-backed decode that prefetches them (outputs
bitwise equal to resident decode, decisions equal to the oracle's LRU run with
the same bets), and the ring's claim histogram (the popularity prewarm's
input)."""
from collections import Counter

import numpy as np
import pytest
import torch

import oracle
import quantised_routed_expert_amd as smoe
import synth
from synth.device import DeviceStack
from tests.gpu_common import need_gpu, random_residual, say
from tests.test_gpu_ring import make_ring, resident_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    torch.cuda.init()


def full_ranking(logits):
    """Expert ids by descending logit, equal logits to the lower index."""
    return sorted(range(len(logits)), key=lambda e: (-logits[e], e))


@pytest.mark.parametrize("dims,n_tok,n_next", [(synth.Dims(256, 128, 128, 8, 32), 5, 8),
                                               (synth.Dims(256, 128, 16, 4, 32), 64, 12),
                                               (synth.Dims(512, 256, 64, 8, 64), 1, 3)])
def test_route_ext_ranks_past_k_match_oracle(dims, n_tok, n_next):
    stack = DeviceStack(1337, dims, 1)
    res = random_residual(np.random.default_rng(n_tok), n_tok, dims.d_model, scale=1.5)
    r = torch.from_numpy(res.copy()).cuda()
    x = torch.empty((n_tok, dims.d_model), dtype=torch.int16, device="cuda")
    idx = torch.empty((n_tok, dims.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((n_tok, dims.top_k), dtype=torch.float32, device="cuda")
    nxt = torch.full((n_tok, n_next), -1, dtype=torch.int32, device="cuda")
    smoe.route_ext(dims, r, x, stack.router_layer(0), None, idx, w, nxt, smoe.workspace(dims, n_tok))
    torch.cuda.synchronize()
    for t in range(n_tok):
        xv, _ = oracle.rmsnorm_bf16(res[t].astype(np.float64), dims.rms_eps)
        rank = full_ranking(oracle.router_logits(stack.router_bits[0], xv))
        assert idx.cpu().numpy()[t].tolist() == rank[: dims.top_k]
        assert nxt.cpu().numpy()[t].tolist() == rank[dims.top_k: dims.top_k + n_next], f"token {t}"


def spec_decode(dims, stack, ring, hidden, n_next):
    """Ring-backed decode that, after each layer, bets on the current token's
    ranks k .. k + n_next - 1 for the next token at that layer."""
    ws = smoe.workspace(dims, 1)
    x = torch.empty((1, dims.d_model), dtype=torch.int16, device="cuda")
    idx = torch.empty((1, dims.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, dims.top_k), dtype=torch.float32, device="cuda")
    nxt = torch.empty((1, n_next), dtype=torch.int32, device="cuda")
    trace, outs = [], []
    for h in hidden:
        r = torch.from_numpy(h.reshape(1, -1).copy()).cuda()
        for L in range(stack.n_layers):
            smoe.route_ext(dims, r, x, stack.router_layer(L), None, idx, w, nxt, ws)
            experts = idx.cpu().numpy()[0].tolist()
            bets = nxt.cpu().numpy()[0].tolist()
            ptrs = ring.acquire(L, experts)
            smoe.moe_decode_slots(dims, x, w, ptrs, r, ws)
            ring.prefetch(L, bets)
            trace.append((L, experts, bets))
        outs.append(r.cpu().numpy()[0])
    ring.release()
    return trace, np.stack(outs)


@pytest.mark.parametrize("n_slots,n_next", [(64, 8), (96, 4)])
def test_ring_prefetch_matches_resident_and_oracle(n_slots, n_next):
    dims = synth.Dims(256, 128, 128, 8, 32)
    n_layers, n_tok = 5, 10
    stack = DeviceStack(1337, dims, n_layers)
    hidden = synth.markov_hidden(1337, n_tok, dims.d_model)
    ring, keep = make_ring(dims, stack, n_slots, pageable_layers={2})
    trace, got = spec_decode(dims, stack, ring, hidden, n_next)
    log = ring.log(1 << 20)
    stats = ring.stats()
    ring.destroy()
    ref = oracle.LruRing(n_slots)
    ref_events = []
    for L, experts, bets in trace:
        ref.release()
        ref_events.extend(ref.acquire(L, experts))
        ref_events.extend(ref.prefetch(L, bets))
    assert log == ref_events
    assert (stats["hits"], stats["misses"], stats["evictions"]) == (ref.hits, ref.misses, ref.evictions)
    assert stats["h2d_bytes"] == (ref.misses + ref.prefetches) * stack.blob_bytes
    say(f"[spec] slots={n_slots} next={n_next}: hits {ref.hits} misses {ref.misses} bets loaded {ref.prefetches}")
    assert np.array_equal(got, resident_decode(dims, stack, hidden))


def test_ring_hottest_counts_every_demand_claim():
    dims = synth.Dims(256, 128, 16, 4, 32)
    n_layers = 3
    stack = DeviceStack(1337, dims, n_layers)
    ring, keep = make_ring(dims, stack, 64)
    rng = np.random.default_rng(3)
    counts = Counter()
    for _ in range(30):
        L = int(rng.integers(n_layers))
        experts = [int(e) for e in rng.choice(dims.n_experts, 4, replace=False, p=None)]
        ring.acquire(L, experts)
        counts.update((L, e) for e in experts)
    ring.prefetch(0, [0, 1, 2])          # bets are not claims
    torch.cuda.synchronize()
    top = ring.hottest(10)
    want = sorted(counts.items(), key=lambda kv: (-kv[1], kv[0][0], kv[0][1]))[:10]
    assert top == [(L, e, c) for (L, e), c in want]
    assert len(ring.hottest(1000)) == len(counts)
    ring.release()
    ring.destroy()
