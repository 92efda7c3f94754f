"""The HBM expert ring on the GPU: its hit/miss/eviction log must equal the
oracle's LRU simulation of the same routing trace, and ring-backed decode and
ring-backed prefill must be bitwise equal to the same work with every expert
resident."""
import numpy as np
import pytest
import torch

import oracle
import quantised_routed_expert_amd as smoe
import synth
from synth.device import DeviceStack, router_stack, u16_to_device
from tests.gpu_common import need_gpu, random_residual, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    torch.cuda.init()


def make_ring(dims, stack, n_slots, log_capacity=1 << 20, pageable_layers=()):
    """A ring over a host copy of the stack's vault: page-locked memory, except
    for the layers in ``pageable_layers`` (ordinary memory, filled through the
    ring's staging pipeline)."""
    stride = stack.stride
    host = torch.empty(stack.vault.numel(), dtype=torch.uint8, pin_memory=True)
    host.copy_(stack.vault)
    plain = torch.empty(stack.vault.numel(), dtype=torch.uint8)
    plain.copy_(stack.vault)
    slab = torch.empty(n_slots * stride, dtype=torch.uint8, device="cuda")
    copy_stream = torch.cuda.Stream()
    per_layer = dims.n_experts * stride
    ptrs = [(plain if L in pageable_layers else host).data_ptr() + L * per_layer for L in range(stack.n_layers)]
    ring = smoe.Ring(n_slots, stack.n_layers, dims.n_experts, dims.top_k, stack.blob_bytes, stride, ptrs, stride,
                     slab.data_ptr(), copy_stream, log_capacity)
    return ring, (host, plain, slab, copy_stream)


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


def test_ring_lru_at_full_scale_with_markov_routing():
    """The ring at the 235B ring workload's scale: 94 layers x 128 experts,
    top-8, 1536 slots, every layer's router input its own Markov chain over
    tokens (0.7 previous + 0.3 fresh), routing done on the GPU at d_model 4096.
    The hit/miss/eviction log must equal the oracle's LRU simulation, and every
    slot must end up holding its key's vault bytes.  The slots carry 4 KiB
    stand-in blobs: the policy and the copies do not depend on blob size."""
    dims = synth.Dims(4096, 1536, 128, 8, 64)
    NL, T, n_slots, E, k = 94, 48, 1536, 128, 8
    blob = 4096
    routers = u16_to_device(router_stack(1337, dims, NL))
    vault = torch.empty((NL, E, blob), dtype=torch.uint8, pin_memory=True)
    vault.copy_(torch.from_numpy(np.random.default_rng(5).integers(0, 256, (NL, E, blob), dtype=np.uint8)))
    slab = torch.full((n_slots, blob), 0, dtype=torch.uint8, device="cuda")
    copy_stream = torch.cuda.Stream()
    ring = smoe.Ring(n_slots, NL, E, k, blob, blob, [vault[L].data_ptr() for L in range(NL)], blob,
                     slab.data_ptr(), copy_stream, NL * T * k)
    hidden = torch.from_numpy(np.stack([synth.markov_hidden(1337, T, dims.d_model, lane=L)
                                        for L in range(NL)])).cuda()
    ws = smoe.workspace(dims, 1)
    x = torch.empty((1, dims.d_model), dtype=torch.int16, device="cuda")
    idx = torch.empty((1, k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, k), dtype=torch.float32, device="cuda")
    routing, repeats = [], []
    for t in range(T):
        layers = []
        for L in range(NL):
            smoe.route(dims, hidden[L, t:t + 1], x, routers[L], None, idx, w, ws)
            experts = idx.cpu().numpy()[0].tolist()
            layers.append(experts)
            if t:
                repeats.append(len(set(experts) & set(routing[-1][L])) / k)
            ring.acquire(L, experts)
        routing.append(layers)
    ring.release()
    torch.cuda.synchronize()
    log = ring.log(NL * T * k)
    stats = ring.stats()
    ring.destroy()
    ref_events, (h, m, ev) = oracle.ring_trace(routing, n_slots)
    assert [e[1:] for e in ref_events] == log
    assert (stats["hits"], stats["misses"], stats["evictions"]) == (h, m, ev)
    say(f"[ring-full] hits {h} misses {m} evictions {ev}, repeat {np.mean(repeats):.3f}")
    assert ev > 0                      # the workload overflows the ring
    holder = {}
    for (_, L, _, e, kind, slot, _) in ref_events:
        if kind == 1:
            holder[slot] = (L, e)
    got = slab.cpu()
    for slot, (L, e) in holder.items():
        assert torch.equal(got[slot], vault[L, e]), (slot, L, e)
    # a sample of the GPU routing against the oracle
    for t, L in ((0, 0), (T - 1, NL - 1), (T // 2, 40)):
        xv, _ = oracle.rmsnorm_bf16(hidden[L, t].cpu().numpy().astype(np.float64), dims.rms_eps)
        ref_idx, _ = oracle.select_topk(oracle.router_logits(synth.router_bits(1337, dims, L), xv), k)
        assert routing[t][L] == ref_idx


def prefill_layers(dims, stack, chunk, ring=None):
    """Layer-major prefill of one chunk through every layer of the stack, each
    layer fed the chunk's own residual (as the prefill workload does).  With a
    ring, the library forms each layer's expert union from the routing and
    acquires it in first-touch order (smoe_ring_acquire_routed), and the GEMMs
    find the blobs through the ring's table; the oracle's union only checks
    it.  Returns the per-layer outputs and unions."""
    T = chunk.shape[0]
    E, k = dims.n_experts, dims.top_k
    ws = smoe.workspace(dims, T)
    x = torch.empty((T, dims.d_model), dtype=torch.int16, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    mu = min(E, T * k)
    uids = torch.empty(mu, dtype=torch.int32, device="cuda")
    ucount = torch.zeros(1, dtype=torch.int32, device="cuda")
    offs = torch.empty(mu + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    table = torch.empty(E, dtype=torch.int64, device="cuda")
    outs, unions = [], []
    for L in range(stack.n_layers):
        r = torch.from_numpy(chunk.copy()).cuda()
        smoe.route(dims, r, x, stack.router_layer(L), stack.bias_layer(L), idx, w, ws)
        if ring is None:
            tab = stack.table(L)
            union = oracle.expert_union(idx.cpu().numpy().tolist())[0]   # synchronises with the router
        else:
            union = ring.acquire_routed(L, idx, table)
            assert union == oracle.expert_union(idx.cpu().numpy().tolist())[0]
            tab = table
        unions.append(union)
        smoe.moe_prefill_chunk(dims, x, idx, w, tab, r, uids, ucount, offs, perm, ws)
        torch.cuda.synchronize()
        assert uids.cpu().numpy()[: int(ucount.item())].tolist() == union
        outs.append(r.cpu().numpy())
    return outs, unions


@pytest.mark.parametrize("bits,n_slots", [(4, 64), (4, 150), (2, 64)])
def test_ring_backed_prefill_matches_resident_and_oracle_log(bits, n_slots):
    """Ring-backed layer-major prefill: acquisitions are whole chunk unions
    (up to min(E, n_slots) experts, fills issued in first-touch order), on
    SMOE-Q4 and SMOE-Q2 blobs."""
    dims = synth.Dims(256, 128, 64, 4, 32) if bits == 4 else synth.Dims(512, 128, 64, 4, 64, bits=2)
    n_layers, T = 4, 20
    stack = DeviceStack(1337, dims, n_layers, zipf_s=1.1)
    rng = np.random.default_rng(5)
    chunks = [random_residual(rng, T, dims.d_model, scale=1.5) for _ in range(3)]
    ring, keep = make_ring(dims, stack, n_slots)
    ref = oracle.LruRing(n_slots)
    ref_events = []
    for c, chunk in enumerate(chunks):
        got, unions = prefill_layers(dims, stack, chunk, ring)
        want, unions_res = prefill_layers(dims, stack, chunk)
        assert unions == unions_res
        for L in range(n_layers):
            assert np.array_equal(got[L], want[L]), f"chunk {c} layer {L}"
            ref.release()
            ref_events.extend(ref.acquire(L, unions[L]))
    log = ring.log(1 << 20)
    stats = ring.stats()
    ring.release()
    ring.destroy()
    assert log == ref_events
    assert (stats["hits"], stats["misses"], stats["evictions"]) == (ref.hits, ref.misses, ref.evictions)
    assert stats["h2d_bytes"] == ref.misses * stack.blob_bytes
    say(f"[ring-prefill] slots={n_slots}: unions {[len(u) for u in unions]}, hits {ref.hits} misses {ref.misses} "
        f"evictions {ref.evictions}")


def test_ring_acquire_routed_rejects_bad_arguments():
    dims = synth.Dims(256, 128, 128, 8, 32)
    stack = DeviceStack(1337, dims, 1)
    ring, keep = make_ring(dims, stack, 64)
    table = torch.empty(dims.n_experts, dtype=torch.int64, device="cuda")
    idx = torch.arange(65 * 8, dtype=torch.int32, device="cuda").reshape(65, 8) % dims.n_experts
    with pytest.raises(smoe.SmoeError):
        ring.acquire_routed(0, idx, table)                       # 65 tokens
    with pytest.raises(smoe.SmoeError):
        ring.acquire_routed(0, idx[:16], table)                  # a union of 128 experts > 64 slots
    with pytest.raises(smoe.SmoeError):
        ring.acquire_routed(1, idx[:2], table)                   # layer out of range
    bad = torch.full((2, 8), dims.n_experts, dtype=torch.int32, device="cuda")
    with pytest.raises(smoe.SmoeError):
        ring.acquire_routed(0, bad, table)                       # no valid expert
    assert ring.acquire_routed(0, idx[:2], table) == list(range(16))
    ring.release()
    ring.destroy()


def test_ring_acquire_table_rejects_oversized_unions():
    dims = synth.Dims(256, 128, 128, 8, 32)
    stack = DeviceStack(1337, dims, 1)
    ring, keep = make_ring(dims, stack, 64)
    table = torch.empty(dims.n_experts, dtype=torch.int64, device="cuda")
    with pytest.raises(smoe.SmoeError):
        ring.acquire_table(0, list(range(65)), table)   # more experts than slots
    ring.acquire_table(0, list(range(64)), table)       # a full ring is fine
    torch.cuda.synchronize()
    t = table.cpu().numpy()
    assert (t[:64] != 0).all() and (t[64:] == 0).all()
    ring.release()
    ring.destroy()


def test_ring_with_pageable_layers_matches_resident():
    """Layers in ordinary (pageable) host memory are filled through the ring's
    staging buffers; decode and prefill through such a ring equal the resident
    results, and the decisions still equal the oracle's."""
    dims = synth.Dims(256, 128, 64, 4, 32)
    n_layers, n_tok, n_slots = 4, 10, 64
    stack = DeviceStack(1337, dims, n_layers, zipf_s=1.1)
    hidden = synth.markov_hidden(1337, n_tok, dims.d_model)
    ring, keep = make_ring(dims, stack, n_slots, pageable_layers={1, 3})
    routing, got = ring_decode(dims, stack, ring, hidden)
    assert np.array_equal(got, resident_decode(dims, stack, hidden))
    chunk = random_residual(np.random.default_rng(9), 24, dims.d_model, scale=1.5)
    pg, unions = prefill_layers(dims, stack, chunk, ring)
    pr, _ = prefill_layers(dims, stack, chunk)
    for L in range(n_layers):
        assert np.array_equal(pg[L], pr[L]), f"prefill layer {L}"
    log = ring.log(1 << 20)
    ring.release()
    ring.destroy()
    ref = oracle.LruRing(n_slots)
    ref_events = []
    for layers in routing:
        for L, experts in enumerate(layers):
            ref.release()
            ref_events.extend(ref.acquire(L, experts))
    for L in range(n_layers):
        ref.release()
        ref_events.extend(ref.acquire(L, unions[L]))
    assert log == ref_events
