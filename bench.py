"""Benchmark: MoE decode tokens/s and achieved HBM GB/s on Q4 expert bytes,
Qwen3-235B-A22B-shaped synthetic stack (94 MoE layers, d_model 4096, expert
ffn 1536, 128 experts, top-8, Q4 chunks of 64), batch 1, all experts resident
in HBM.

A step is one decode token through all 94 layers: exact routing (RMSNorm,
float64 gate matvec, top-8, norm_topk_prob) and the fused SMOE-Q4 expert FFN
added into the residual, each step starting from a fresh N(0,1) bf16 hidden
state.  The token's 282 kernels are captured once into a HIP graph and
replayed; the step's input copy runs eagerly inside the timed region.  The
line also carries ``prefill``: the prefill workload (a 512-token prompt in
chunks of 64, Zipf(1.1)-biased routing) on the same stack (same experts and
routers), with its own roofline (union bytes over grouped-GEMM time), MFMA
utilisation and oracle baseline.  Prefill keeps four chunks in flight on four
streams, each one layer behind the previous and waiting for it layer by layer
(``--chunks-in-flight``; the one-chunk time is reported beside it).

Other workloads (one JSON line each): ``--workload prefill`` -- a 512-token
prompt in chunks of 64 through the same 94 layers, layer-major, Zipf-biased
routing; ``--workload ring`` -- decode with the experts in a 1536-slot HBM ring
refilled from a vault in pinned host memory (Markov hidden states).

Prints one JSON line.  ``--gpus N`` with N > 1 is refused: the layer is built and measured on
one GPU.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import ctypes  # noqa: E402

import numpy as np  # noqa: E402
import torch  # noqa: E402

import quantised_routed_expert_amd as smoe  # noqa: E402
import synth  # noqa: E402
from synth.device import DeviceStack  # noqa: E402

HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_FLOPS = 2.5e15  # MI355X dense fp16 / bf16 matrix peak
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000
# sources of the decode gate/up kernel: a stored traffic figure counts only
# while they are unchanged since its counters were read
GATE_UP_SOURCES = ("quantised_routed_expert_amd/csrc/decode.hip", "quantised_routed_expert_amd/csrc/kernels.h",
                   "quantised_routed_expert_amd/csrc/smoe_internal.h")
TRAFFIC_FILES = {("235b", 4): "profiles/hbm_traffic_decode_gate_up_235b.txt",
                 ("235b", 2): "profiles/hbm_traffic_decode_gate_up_235b_q2.txt",
                 ("30b", 4): "profiles/hbm_traffic_decode_gate_up_30b.txt",
                 ("30b", 2): "profiles/hbm_traffic_decode_gate_up_30b_q2.txt"}
# decode stacks by (shape, code width)
DECODE_WORKLOADS = {("235b", 4): synth.CONFIGS[2], ("235b", 2): synth.Q2_WORKLOADS[0],
                    ("30b", 4): synth.CONFIGS[1], ("30b", 2): synth.Q2_WORKLOADS[2]}
SHAPE_LABEL = {"235b": "235B-shape", "30b": "30B-shape"}


def sources_digest(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(bits=4, shape="235b"):
    """HBM bytes per gate/up launch from the committed counter summary (FETCH_SIZE
    + WRITE_SIZE, each scaled by the copy-kernel calibration) for the decode
    stack ``shape`` at code width ``bits``, or None if there is none or the
    kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, TRAFFIC_FILES[(shape, bits)])
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != sources_digest(GATE_UP_SOURCES):
        log("stored traffic figure is stale (kernel sources changed): traffic = null")
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles (the library records them on its own stream)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p(0)
            # timing-only events: no system-scope fence (no L2 writeback and
            # invalidate around the timed kernel)
            assert self.hip.hipEventCreateWithFlags(ctypes.byref(h), HIP_EVENT_DISABLE_SYSTEM_FENCE) == 0
            self.ev.append(h.value)

    def elapsed_ms(self, a, b):
        out = ctypes.c_float(0)
        rc = self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(self.ev[a]),
                                          ctypes.c_void_p(self.ev[b]))
        assert rc == 0, rc
        return float(out.value)

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def read_references(per_launch, instrument_steps):
    """Attainable read bandwidth, from the plain streaming-read kernel in
    synth/probe.hip: (a) over a 4 GiB buffer, far beyond the 256 MB MALL;
    (b) one launch over ``per_launch`` bytes, each launch on a different
    region of that buffer, timed like the gate/up kernel (hipExtLaunchKernel
    events, queue pre-filled).  Returns GB/s for both."""
    from synth.device import stream_read
    big = 4 << 30
    buf = torch.empty(big, dtype=torch.uint8, device="cuda")
    sink = torch.empty(1024, dtype=torch.int32, device="cuda")
    n_big = 10
    ev = HipEvents(2 * n_big)
    for _ in range(2):
        stream_read(buf, big, sink=sink)
    torch.cuda._sleep(5_000_000)
    for i in range(n_big):
        stream_read(buf, big, sink=sink, start=ev.ev[2 * i], stop=ev.ev[2 * i + 1])
    torch.cuda.synchronize()
    big_ms = float(np.mean([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(n_big)]))
    ev.close()
    per = (per_launch + 255) // 256 * 256
    regions = big // per
    n_small = max(1, min(regions, 8 * instrument_steps))
    ev = HipEvents(2 * n_small)
    torch.cuda._sleep(5_000_000)
    for i in range(n_small):
        stream_read(buf, per_launch, offset=i * per, sink=sink, start=ev.ev[2 * i], stop=ev.ev[2 * i + 1])
    torch.cuda.synchronize()
    small_ms = float(np.mean([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(n_small)]))
    ev.close()
    del buf
    return {"stream_4gib_gbps": big / (big_ms / 1e3) / 1e9,
            "one_launch_same_bytes_gbps": per_launch / (small_ms / 1e3) / 1e9,
            "one_launch_same_bytes_us": small_ms * 1e3}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(stack, wl, budget_s=15.0):
    """The float64 oracle on the host cores: one token through as many of the
    stack's layers as fit in ``budget_s`` of oracle time (input drawing is not
    timed), extrapolated to tokens/s over all layers."""
    import oracle
    from threadpoolctl import threadpool_info
    dims = wl.dims
    r = synth.hidden_bf16(wl.seed, 10_000, dims.d_model).astype(np.float64)
    spent, n = 0.0, 0
    for L in range(wl.n_layers):
        t0 = time.perf_counter()
        x, _ = oracle.rmsnorm_bf16(r, dims.rms_eps)
        idx, w = oracle.select_topk(oracle.router_logits(stack.router_bits[L], x), dims.top_k,
                                    dims.norm_topk_prob)
        t1 = time.perf_counter()
        experts = [synth.expert_logical(wl.seed, dims, L, e) for e in idx]
        t2 = time.perf_counter()
        y = np.zeros(dims.d_model)
        for rk in range(dims.top_k):
            y = y + w[rk] * oracle.expert_ffn(experts[rk], x, dims.chunk)
        r = r + y
        t3 = time.perf_counter()
        spent += (t1 - t0) + (t3 - t2)
        n += 1
        if spent >= budget_s:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    per_token = spent / n * wl.n_layers
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": os.cpu_count(), "blas_threads": threads,
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"1 decode token through the first {n} of {wl.n_layers} layers, float64 numpy oracle, "
                      f"{spent:.1f} s of oracle time; tokens/s extrapolated to all {wl.n_layers} layers"}


def bench_decode(args):
    wl = DECODE_WORKLOADS[(args.shape, 4 if args.quant == "q4" else 2)]
    dims = wl.dims
    qname = args.quant.upper()
    torch.cuda.set_device(0)
    t0 = time.time()
    stack = DeviceStack(wl.seed, dims, wl.n_layers)
    torch.cuda.synchronize()
    log(f"stack ready in {time.time() - t0:.1f} s: vault {stack.vault.numel() / 1e9:.2f} GB")

    K, W = args.steps, args.warmup
    hid = np.stack([synth.hidden_bf16(wl.seed + 1, i, dims.d_model) for i in range(W)] +
                   [synth.hidden_bf16(wl.seed, i, dims.d_model) for i in range(K)])
    H = torch.from_numpy(hid).cuda()
    resid = torch.empty(dims.d_model, dtype=torch.float32, device="cuda")
    ws = smoe.workspace(dims, 1)

    # capture one token (all layers) into a graph
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        resid.copy_(H[0])
        smoe.decode_layers(dims, wl.n_layers, resid, stack.router, None, stack.tables, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        smoe.decode_layers(dims, wl.n_layers, resid, stack.router, None, stack.tables, ws)
    torch.cuda.synchronize()

    for i in range(W):
        resid.copy_(H[i])
        g.replay()
    torch.cuda.synchronize()
    log("warmup done")

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(K):
        resid.copy_(H[W + i])
        g.replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    tok_s = K / (ms / 1000.0)
    log(f"timed {K} steps: {ms:.3f} ms, {tok_s:.1f} tokens/s")

    # per-kernel timing of the gate/up kernel (the dominant kernel): the same
    # token launched eagerly with hipExtLaunchKernel start/stop events on the
    # library's stream.  A spin kernel ahead of it keeps the GPU busy while the
    # host enqueues all of the token's launches, so they then run back to back
    # as in the graph replays above.
    off = synth.blob_sections(dims)
    gate_up_bytes = (off["down_codes"] - off["gate_codes"]) + (off["down_params"] - off["gate_params"])
    per_launch = dims.top_k * gate_up_bytes
    ev = HipEvents(2 * wl.n_layers)
    durs = []
    for i in range(args.instrument_steps):
        resid.copy_(H[W + i % K])
        torch.cuda._sleep(20_000_000)
        smoe.decode_layers(dims, wl.n_layers, resid, stack.router, None, stack.tables, ws, events=ev.ev)
        torch.cuda.synchronize()
        durs += [ev.elapsed_ms(2 * L, 2 * L + 1) for L in range(wl.n_layers)]
    ev.close()
    gu_ms = float(np.mean(durs))
    achieved = per_launch / (gu_ms / 1000.0) / 1e9
    log(f"gate/up kernel: {gu_ms * 1000:.2f} us avg over {len(durs)} launches, {achieved:.0f} GB/s")
    refs = read_references(per_launch, args.instrument_steps)
    log(f"plain reads: 4 GiB stream {refs['stream_4gib_gbps']:.0f} GB/s; one launch of the same "
        f"{per_launch} B {refs['one_launch_same_bytes_us']:.2f} us = {refs['one_launch_same_bytes_gbps']:.0f} GB/s")

    layer_bytes = dims.top_k * off["bytes"] + dims.n_experts * dims.d_model * 2
    bytes_per_token = wl.n_layers * layer_bytes
    layer_us = ms / K * 1000.0 / wl.n_layers
    out = {
        "metric": f"MoE decode tokens/s + achieved HBM GB/s on {qname} expert bytes ({SHAPE_LABEL[args.shape]})",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{args.quant}-affine weights, f16 dot products with fp32 accumulation; float64 router",
        "data": "synthetic (seeded SplitMix64 codes/scales, N(0,0.02) router, N(0,1) bf16 hidden states)",
        "config": {"workload": wl.name, "layers": wl.n_layers, "d_model": dims.d_model, "d_ff": dims.d_ff,
                   "experts": dims.n_experts, "top_k": dims.top_k, "chunk": dims.chunk, "code_bits": dims.bits,
                   "batch": 1,
                   "vault_bytes": stack.vault.numel(), "parallelism": "single GPU"},
        f"gbps_{args.quant}_expert_and_router_bytes": tok_s * bytes_per_token / 1e9,
        "per_layer": {"bytes": layer_bytes, "us": layer_us, "gbps": layer_bytes / layer_us / 1e3,
                      "frac": layer_bytes / layer_us / 1e3 / HBM_PEAK_GBPS,
                      "timing": "graph replays: token time / layers; a layer's three kernels and the next "
                                "layer's run back to back, so this is one layer's first-kernel start to "
                                "last-kernel end plus one launch gap"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": stored_traffic(dims.bits, args.shape),
                     "kernel": "decode_gate_up_kernel", "bytes_per_launch": per_launch,
                     "avg_launch_us": gu_ms * 1000.0, "launches_timed": len(durs),
                     "timing": "hipExtLaunchKernel start/stop events, eager token with the queue pre-filled",
                     "attainable": dict(refs, frac_of_stream_4gib=achieved / refs["stream_4gib_gbps"],
                                        frac_of_one_launch_same_bytes=achieved
                                        / refs["one_launch_same_bytes_gbps"])},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(stack, wl, args.cpu_budget)
    pwl = PREFILL_WORKLOADS.get(dims.bits)
    if args.shape == "235b" and not args.no_prefill and pwl is not None and vars(pwl.dims) == vars(dims) \
            and pwl.seed == wl.seed and pwl.n_layers == wl.n_layers:
        # the prefill workload has the same experts and routers: only its Zipf
        # logit bias is new
        log("prefill on the same stack ...")
        del H, ws, g
        bias = torch.from_numpy(np.stack([synth.zipf_bias(pwl.seed, dims, L, pwl.zipf_s)
                                          for L in range(pwl.n_layers)])).cuda()
        out["prefill"] = measure_prefill(stack, pwl, pwl.n_layers, bias, args.prefill_steps, 1, chained=False,
                                         lanes=args.chunks_in_flight,
                                         cpu_budget=None if args.no_cpu_baseline else args.prefill_cpu_budget)
    print(json.dumps(out), flush=True)


def graph_of(fn):
    """Run ``fn`` once eagerly on a side stream (warm-up), then capture it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_replays(g, warmup, steps, before=None):
    for i in range(warmup):
        if before:
            before(i)
        g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        if before:
            before(warmup + i)
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


PREFILL_WORKLOADS = {4: synth.CONFIGS[3], 2: synth.Q2_WORKLOADS[3]}


def prefill_cpu_baseline(stack, wl, bias_np, prompt_np, budget_s=10.0):
    """The float64 oracle on the host cores for the prefill workload: the first
    tokens of the prompt's first chunk through layer 0 (oracle.moe_layer per
    token, as oracle.prefill_chunk runs a chunk), as many as fit in
    ``budget_s`` of oracle time (drawing the experts is not timed); per
    chunk-layer seconds and prompt tokens/s are extrapolated from the
    per-token time."""
    import oracle
    from threadpoolctl import threadpool_info
    dims = wl.dims
    cache = {}

    class Experts(dict):
        def __missing__(self, e):
            cache[e] = synth.expert_logical(wl.seed, dims, 0, e)
            return cache[e]

    experts = Experts()
    spent, n = 0.0, 0
    for t in range(wl.prefill_chunk):
        r = prompt_np[t].astype(np.float64)
        x, _ = oracle.rmsnorm_bf16(r, dims.rms_eps)
        idx, _ = oracle.select_topk(oracle.router_logits(stack.router_bits[0], x, bias_np[0]), dims.top_k,
                                    dims.norm_topk_prob)
        for e in idx:  # draw the token's experts outside the timed region
            experts[int(e)]
        t0 = time.perf_counter()
        oracle.moe_layer(r, stack.router_bits[0], experts, dims, bias_np[0])
        spent += time.perf_counter() - t0
        n += 1
        if spent >= budget_s:
            break
    per_token_layer = spent / n
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": 1.0 / (per_token_layer * wl.n_layers), "unit": "prompt tokens/s", "cores": os.cpu_count(),
            "blas_threads": threads, "kind": "oracle", "cpu": cpu_model(),
            "s_per_chunk_layer": per_token_layer * wl.prefill_chunk,
            "sample": f"the first {n} tokens of chunk 0 through layer 0 (float64 numpy oracle.moe_layer, "
                      f"{spent:.1f} s of oracle time); per chunk-layer = per token x {wl.prefill_chunk}, "
                      f"prompt tokens/s = 1 / (per token x {wl.n_layers} layers)"}


def measure_prefill(stack, wl, NL, bias, steps, warmup, chained=True, instrument_chunks=2, cpu_budget=None,
                    lanes=1, graph=True):
    """Layer-major prefill of the workload's prompt in chunks through NL layers
    of ``stack`` (router logits biased by ``bias`` [NL][E]): for each chunk and
    layer, route the chunk, build the expert union, run the grouped expert FFN
    and combine into the residual.

    Two readings of the per-layer input are timed.  ``fresh`` (the reported
    one): every layer's MoE input is the prompt's own N(0,1) hidden state (the
    layers' routers and Zipf permutations are independent, so each layer sees
    realistic unions).  ``chained``: layer L+1 reads layer L's output residual;
    with the synthetic weights (mean -scale/2 per element) the residual drifts
    to one common direction within ~10 layers and every token then routes
    alike, so the unions collapse.

    ``lanes`` > 1 keeps that many chunks in flight on as many streams: chunk c
    runs on stream c % lanes, one layer behind chunk c - 1, and its layer L
    waits for chunk c - 1's layer L (the order a causal model needs: a
    chunk's layer reads the earlier chunks' output of that layer).  One
    chunk's latency-bound routing and union kernels then overlap another's
    grouped GEMMs.  Each stream has its own routing buffers and workspace.

    Kernel timing: the first ``instrument_chunks`` chunks through all NL layers
    are run eagerly with start/stop events around the two grouped GEMMs (the
    queue pre-filled by a spin kernel); the roofline is union bytes over GEMM
    time."""
    dims = wl.dims
    T, C = wl.steps, wl.prefill_chunk
    n_chunks = T // C
    prompt_np = np.stack([synth.hidden_bf16(wl.seed, 20_000 + t, dims.d_model) for t in range(T)])
    prompt = torch.from_numpy(prompt_np).cuda()
    resid = torch.empty_like(prompt)
    mu = min(dims.n_experts, C * dims.top_k)
    ucount = {m: torch.zeros((n_chunks, NL), dtype=torch.int32, device="cuda")
              for m in ("fresh", "chained", "fresh_one_lane", "ev")}

    def lane_buffers():
        return {"x": torch.empty((C, dims.d_model), dtype=torch.int16, device="cuda"),
                "idx": torch.empty((C, dims.top_k), dtype=torch.int32, device="cuda"),
                "w": torch.empty((C, dims.top_k), dtype=torch.float32, device="cuda"),
                "uids": torch.empty(mu, dtype=torch.int32, device="cuda"),
                "offs": torch.empty(mu + 1, dtype=torch.int32, device="cuda"),
                "perm": torch.empty(C * dims.top_k, dtype=torch.int32, device="cuda"),
                "ws": smoe.workspace(dims, C)}

    lanes = max(1, min(int(lanes), n_chunks))
    bufs = [lane_buffers() for _ in range(lanes)]
    streams = [None] + [torch.cuda.Stream() for _ in range(lanes - 1)]  # default priority

    def layer(L, c, r, uc, events=None):
        b = bufs[c % lanes]
        smoe.route(dims, r, b["x"], stack.router_layer(L), bias[L], b["idx"], b["w"], b["ws"])
        smoe.moe_prefill_chunk(dims, b["x"], b["idx"], b["w"], stack.table(L), r, b["uids"], uc[c, L:L + 1],
                               b["offs"], b["perm"], b["ws"], events=events)

    done = [[torch.cuda.Event() for _ in range(NL)] for _ in range(lanes)] if lanes > 1 else None

    def run_prompt(fresh, uc, nl):
        # groups of nl chunks; within a group chunk c0 + j is j layers behind
        # chunk c0 and waits for chunk c0 + j - 1 to finish each layer
        main = torch.cuda.current_stream()
        for st in streams[1:nl]:
            st.wait_stream(main)
        for c0 in range(0, n_chunks, nl):
            nc = min(nl, n_chunks - c0)
            for step in range(NL + nc - 1):
                for j in range(nc):
                    L, c = step - j, c0 + j
                    if not 0 <= L < NL:
                        continue
                    st = streams[j] or main
                    with torch.cuda.stream(st):
                        if j > 0:
                            st.wait_event(done[j - 1][L])
                        r = resid[c * C:(c + 1) * C]
                        if fresh:
                            r.copy_(prompt[c * C:(c + 1) * C])
                        layer(L, c, r, uc)
                        if done is not None and j + 1 < nc:
                            done[j][L].record(st)
            for st in streams[1:nl]:  # the next group starts after this one
                main.wait_stream(st)

    def prompt_fresh():
        run_prompt(True, ucount["fresh"], lanes)

    def prompt_chained():
        resid.copy_(prompt)
        run_prompt(False, ucount["chained"], lanes)

    def prompt_fresh_one_lane():
        run_prompt(True, ucount["fresh_one_lane"], 1)

    off = synth.blob_sections(dims)
    gate_up_bytes = (off["down_codes"] - off["gate_codes"]) + (off["down_params"] - off["gate_params"])
    down_bytes = off["bytes"] - gate_up_bytes
    flops_per_prompt = 6.0 * dims.d_model * dims.d_ff * dims.top_k * NL * T
    res = {}
    readings = [("fresh", prompt_fresh)] + ([("chained", prompt_chained)] if chained else []) + \
        ([("fresh_one_lane", prompt_fresh_one_lane)] if lanes > 1 else [])
    for mode, fn in readings:
        if graph:
            g = graph_of(fn)
            ms = time_replays(g, warmup, steps)
        else:  # eager launches (the streams of the lanes run as the host issues them)
            g = None
            for _ in range(max(1, warmup)):
                fn()
            torch.cuda.synchronize()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(steps):
                fn()
            t1.record()
            torch.cuda.synchronize()
            ms = t0.elapsed_time(t1) / steps
        u = ucount[mode].cpu().numpy()
        ub = int(u.sum()) * off["bytes"]
        res[mode] = {"ms": ms, "tok_s": T / (ms / 1e3), "mean_union": float(u.mean()),
                     "union_bytes": ub, "union_gbps": ub / (ms / 1e3) / 1e9,
                     "mfma_utilisation": flops_per_prompt / (ms / 1e3) / MFMA_F16_PEAK_FLOPS}
        log(f"prefill[{mode}]: {ms:.2f} ms/prompt, {res[mode]['tok_s']:.0f} tokens/s, "
            f"mean |union| {u.mean():.1f}, {res[mode]['union_gbps']:.0f} GB/s on union bytes")
        del g

    # per-kernel GEMM timing, fed-prompt reading, first chunks
    nc = max(1, min(instrument_chunks, n_chunks))
    ev = HipEvents(4 * nc * NL)
    torch.cuda.synchronize()
    torch.cuda._sleep(50_000_000)
    for c in range(nc):
        r = resid[c * C:(c + 1) * C]
        for L in range(NL):
            r.copy_(prompt[c * C:(c + 1) * C])
            layer(L, c, r, ucount["ev"], events=ev.ev[4 * (c * NL + L):4 * (c * NL + L) + 4])
    torch.cuda.synchronize()
    u = ucount["ev"][:nc].cpu().numpy().reshape(-1)
    gu = np.array([ev.elapsed_ms(4 * i, 4 * i + 1) for i in range(nc * NL)])
    dn = np.array([ev.elapsed_ms(4 * i + 2, 4 * i + 3) for i in range(nc * NL)])
    ev.close()
    gu_gbps = float((u * gate_up_bytes).sum() / (gu.sum() / 1e3) / 1e9)
    dn_gbps = float((u * down_bytes).sum() / (dn.sum() / 1e3) / 1e9)
    gemm_gbps = float((u * off["bytes"]).sum() / ((gu + dn).sum() / 1e3) / 1e9)
    gemm_flops = 6.0 * dims.d_model * dims.d_ff * dims.top_k * C * len(u)
    mfma_gemm = gemm_flops / ((gu + dn).sum() / 1e3) / MFMA_F16_PEAK_FLOPS
    log(f"prefill GEMMs: gate/up {gu.mean() * 1e3:.1f} us ({gu_gbps:.0f} GB/s), down {dn.mean() * 1e3:.1f} us "
        f"({dn_gbps:.0f} GB/s) over {len(u)} chunk-layers, mean |union| {u.mean():.1f}")
    f = res["fresh"]
    out = {
        "value": f["tok_s"], "unit": "prompt tokens/s", "ms_per_prompt": f["ms"],
        "config": {"workload": wl.name, "layers": NL, "prompt_tokens": T, "chunk": C},
        "dtype": f"q{dims.bits}-affine codes as fp16 MFMA inputs, fp32 accumulation with the affine step folded "
                 "per chunk; float64 router",
        "data": "synthetic (seeded SplitMix64 codes/scales, N(0,0.02) router, Zipf(1.1) logit bias, N(0,1) bf16 "
                "prompt hidden states fed to every layer)",
        "mean_union": f["mean_union"], "union_bytes_per_prompt": f["union_bytes"], "union_gbps": f["union_gbps"],
        "union_hbm_frac": f["union_gbps"] / HBM_PEAK_GBPS, "mfma_utilisation": f["mfma_utilisation"],
        "roofline": {"bound": "hbm", "achieved": gu_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gu_gbps / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "prefill grouped gate/up GEMM", "bytes_per_launch": float(u.mean() * gate_up_bytes),
                     "avg_launch_us": float(gu.mean() * 1e3), "launches_timed": int(len(u)),
                     "timing": "hipExtLaunchKernel start/stop events, eager chunks with the queue pre-filled",
                     "down_gemm": {"avg_launch_us": float(dn.mean() * 1e3), "achieved": dn_gbps,
                                   "frac": dn_gbps / HBM_PEAK_GBPS},
                     "both_gemms": {"achieved": gemm_gbps, "frac": gemm_gbps / HBM_PEAK_GBPS,
                                    "mfma_utilisation": mfma_gemm}},
    }
    out["config"]["chunks_in_flight"] = lanes
    if chained:
        out["chained"] = {k: res["chained"][k] for k in ("tok_s", "ms", "mean_union", "union_gbps",
                                                         "mfma_utilisation")}
    if lanes > 1:
        out["one_chunk_in_flight"] = {k: res["fresh_one_lane"][k] for k in ("tok_s", "ms", "union_gbps",
                                                                            "mfma_utilisation")}
    if cpu_budget:
        log("cpu baseline (oracle, prefill) ...")
        out["cpu_baseline"] = prefill_cpu_baseline(stack, wl, bias.cpu().numpy(), prompt_np, cpu_budget)
    return out


def bench_prefill(args):
    """The prefill workload alone: a 512-token prompt in chunks of 64 through
    the 94 layers (see measure_prefill)."""
    wl = PREFILL_WORKLOADS[4 if args.quant == "q4" else 2]
    dims = wl.dims
    NL = wl.n_layers if args.layers is None else max(1, min(args.layers, wl.n_layers))
    torch.cuda.set_device(0)
    stack = DeviceStack(wl.seed, dims, NL, zipf_s=wl.zipf_s)
    torch.cuda.synchronize()
    log(f"stack ready: vault {stack.vault.numel() / 1e9:.2f} GB")
    p = measure_prefill(stack, wl, NL, stack.bias, args.steps, args.warmup, lanes=args.chunks_in_flight,
                        graph=not args.prefill_eager,
                        cpu_budget=None if args.no_cpu_baseline else args.cpu_budget)
    out = {
        "metric": "layer-major prefill prompt tokens/s + GB/s on union expert bytes (235B-shape, 512-token "
                  "prompt, chunks of 64" + (")" if dims.bits == 4 else ", SMOE-Q2)"),
        "value": p.pop("value"), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": p.pop("ms_per_prompt"), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
    }
    p.pop("unit")
    cfg = p.pop("config")
    cfg["parallelism"] = "single GPU"
    out.update(dtype=p.pop("dtype"), data=p.pop("data"), config=cfg)
    out.update(p)
    print(json.dumps(out), flush=True)


def host_vault(wl, args):
    """The expert vault in host memory, one allocation per layer, drawn on the
    device and copied down.  Layers are page-locked (hipHostMalloc) up to
    --pinned-gib; the driver caps page-locked memory (64 GiB on the MI355X
    hosts measured), so the rest of a 128 GB vault stays pageable and its fills
    are staged by the HIP runtime.  Returns (pinned buffers, per-layer views,
    number of page-locked layers)."""
    from synth.device import fill_experts
    dims = wl.dims
    E, NL = dims.n_experts, wl.n_layers
    stride = synth.blob_sections(dims)["stride"]
    t0 = time.time()
    pinned_budget = int(args.pinned_gib * (1 << 30))
    vault, views = [], []
    for L in range(NL):
        buf = None
        if (len(vault) + 1) * E * stride <= pinned_budget:
            try:
                buf = smoe.PinnedHost(E * stride)
            except smoe.SmoeError:
                pinned_budget = 0
        if buf is not None:
            vault.append(buf)
            views.append(buf.tensor())
        else:
            views.append(torch.empty(E * stride, dtype=torch.uint8))
    n_pinned = len(vault)
    stage = torch.empty(E * stride, dtype=torch.uint8, device="cuda")
    for L in range(NL):
        fill_experts(wl.seed, dims, L, 0, E, stage.data_ptr(), stride)
        views[L].copy_(stage)
    del stage
    log(f"vault: {n_pinned} of {NL} layers page-locked ({n_pinned * E * stride / 1e9:.1f} GB), "
        f"drawn in {time.time() - t0:.1f} s")
    return vault, views, n_pinned


def bench_ring(args):
    """Decode with a 1536-slot HBM ring over a vault in pinned host memory.
    Each layer's router input follows its own Markov chain over tokens
    (h_t = 0.7 h_{t-1} + 0.3 z_t), so consecutive tokens share part of their
    experts; the residual update of each layer is computed and discarded."""
    wl = synth.CONFIGS[4] if args.quant == "q4" else synth.Q2_WORKLOADS[1]
    dims = wl.dims
    E, NL = dims.n_experts, wl.n_layers
    torch.cuda.set_device(0)
    off = synth.blob_sections(dims)
    stride = off["stride"]
    t0 = time.time()
    from synth.device import router_stack, u16_to_device
    link = h2d_references()
    log(f"host link: pinned H2D {link['pinned_h2d_gbps']:.1f} GB/s, pageable H2D {link['pageable_h2d_gbps']:.1f} GB/s")
    vault, views, n_pinned = host_vault(wl, args)
    router = u16_to_device(router_stack(wl.seed, dims, NL))
    keep, fresh = wl.markov
    W, K = args.warmup, args.steps
    hidden = torch.from_numpy(np.stack([synth.markov_hidden(wl.seed, W + K, dims.d_model, keep, fresh, lane=L)
                                        for L in range(NL)])).cuda()          # [L][t][d]
    log(f"vault and Markov states drawn in {time.time() - t0:.1f} s")
    n_slots = wl.ring_slots
    slab = torch.empty(n_slots * stride, dtype=torch.uint8, device="cuda")
    copy_stream = torch.cuda.Stream()
    ring = smoe.Ring(n_slots, NL, E, dims.top_k, off["bytes"], stride, [v.data_ptr() for v in views], stride,
                     slab.data_ptr(), copy_stream, 0)
    ws = smoe.workspace(dims, 1)
    x = torch.empty((1, dims.d_model), dtype=torch.int16, device="cuda")
    idx = torch.empty((1, dims.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, dims.top_k), dtype=torch.float32, device="cuda")
    S = args.spec
    sel = torch.empty((1, dims.top_k + S), dtype=torch.int32, device="cuda")   # ranks 0 .. k + S - 1
    sel_host = torch.empty((1, dims.top_k + S), dtype=torch.int32, pin_memory=True)
    r = torch.empty((1, dims.d_model), dtype=torch.float32, device="cuda")
    prev = [None] * NL
    repeats = []
    bets_loaded = [0]

    def token(t, count):
        for L in range(NL):
            r.copy_(hidden[L, t:t + 1])
            if S:
                smoe.route_ext(dims, r, x, router[L], None, sel[:, :dims.top_k], w, sel[:, dims.top_k:], ws)
            else:
                smoe.route(dims, r, x, router[L], None, sel, w, ws)
            sel_host.copy_(sel)
            torch.cuda.current_stream().synchronize()
            ranked = sel_host.numpy()[0].tolist()
            experts = ranked[:dims.top_k]
            if count and prev[L] is not None:
                repeats.append(len(set(experts) & set(prev[L])) / dims.top_k)
            prev[L] = experts
            ptrs = ring.acquire(L, experts)
            smoe.moe_decode_slots(dims, x, w, ptrs, r, ws)
            if S:  # bets on the next token at this layer: this token's ranks k .. k + S - 1
                n = ring.prefetch(L, ranked[dims.top_k:])
                if count:
                    bets_loaded[0] += n

    for t in range(W):
        token(t, False)
    torch.cuda.synchronize()
    prewarm_loads = 0
    if args.prewarm:  # idle time between turns: the historically hottest experts into the ring
        ring.release()
        hot = ring.hottest(n_slots)
        by_layer = {}
        for L, e, _ in hot:
            by_layer.setdefault(L, []).append(e)
        for L in sorted(by_layer):
            prewarm_loads += ring.prefetch(L, by_layer[L])
        torch.cuda.synchronize()
        log(f"prewarm: {prewarm_loads} loads from {len(hot)} hottest (layer, expert) pairs")
    s0 = ring.stats()
    t1 = time.time()
    for t in range(K):
        token(W + t, True)
    torch.cuda.synchronize()
    dt = time.time() - t1
    s1 = ring.stats()
    ring.release()
    ring.destroy()
    hits, misses = s1["hits"] - s0["hits"], s1["misses"] - s0["misses"]
    h2d = s1["h2d_bytes"] - s0["h2d_bytes"]
    tok_s = K / dt
    log(f"ring: {tok_s:.2f} tokens/s, hit rate {hits / max(1, hits + misses):.3f}, "
        f"H2D {h2d / dt / 1e9:.1f} GB/s, repeat {np.mean(repeats):.3f}")
    out = {
        "metric": f"ring-backed MoE decode tokens/s (235B-shape, {n_slots}-slot HBM ring over a pinned-host vault)",
        "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": dt * 1000.0 / K, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"{args.quant}-affine weights, f16 dot products with fp32 accumulation; float64 router",
        "data": "synthetic (per-layer Markov router inputs h_t = 0.7 h_{t-1} + 0.3 z_t)",
        "config": {"workload": wl.name, "layers": NL, "ring_slots": n_slots, "code_bits": dims.bits,
                   "slot_bytes": off["bytes"], "spec": S, "prewarm": bool(args.prewarm),
                   "parallelism": "single GPU"},
        "hit_rate": hits / max(1, hits + misses), "misses_per_token": misses / K,
        "bets_loaded_per_token": bets_loaded[0] / K, "prewarm_loads": prewarm_loads,
        "h2d_gbps": h2d / dt / 1e9, "expert_repeat_fraction": float(np.mean(repeats)),
        "vault_layers_page_locked": n_pinned,
        "host_link": dict(link, h2d_frac_of_pinned=h2d / dt / 1e9 / link["pinned_h2d_gbps"]),
    }
    del views
    for v in vault:
        v.free()
    print(json.dumps(out), flush=True)


def bench_ring_prefill(args):
    """Layer-major prefill through the HBM ring over the host vault (1536 slots for
    SMOE-Q4, 2764 for SMOE-Q2: the same 16.31 GB of HBM):
    the 512-token prompt in chunks of 64 with the Zipf(1.1) logit bias, every
    layer fed the prompt (as the prefill workload does).  Per chunk and layer
    the routing is read back, the expert union is acquired in first-touch
    order (its fills go out on the copy stream in that order, the first-touched
    expert first) and the grouped GEMMs find the blobs through the ring's
    expert table.  One warm-up prompt fills the ring; the timed prompts follow.

    Two schedules, same results: ``value`` takes the chunks in turn, each
    through all layers (the pages' order: a union is read once per chunk);
    ``layer_outer`` takes the layers in turn, each over all chunks, so that a
    layer's union is loaded once and the later chunks hit it in the ring."""
    from synth.device import router_stack, u16_to_device
    wl = synth.CONFIGS[3] if args.quant == "q4" else synth.Q2_WORKLOADS[3]
    dims = wl.dims
    E, NL, k = dims.n_experts, wl.n_layers, dims.top_k
    T, C = wl.steps, wl.prefill_chunk
    n_chunks = T // C
    # the decode ring's slot count for the code width (the same 16.31 GB of HBM)
    n_slots = (synth.CONFIGS[4] if args.quant == "q4" else synth.Q2_WORKLOADS[1]).ring_slots
    torch.cuda.set_device(0)
    off = synth.blob_sections(dims)
    stride = off["stride"]
    link = h2d_references()
    log(f"host link: pinned H2D {link['pinned_h2d_gbps']:.1f} GB/s, pageable H2D {link['pageable_h2d_gbps']:.1f} GB/s")
    vault, views, n_pinned = host_vault(wl, args)
    router = u16_to_device(router_stack(wl.seed, dims, NL))
    bias = torch.from_numpy(np.stack([synth.gen.zipf_bias(wl.seed, dims, L, wl.zipf_s) for L in range(NL)])).cuda()
    prompt = torch.from_numpy(np.stack([synth.hidden_bf16(wl.seed, 20_000 + t, dims.d_model)
                                        for t in range(T)])).cuda()
    resid = torch.empty_like(prompt)
    slab = torch.empty(n_slots * stride, dtype=torch.uint8, device="cuda")
    copy_stream = torch.cuda.Stream()
    ring = smoe.Ring(n_slots, NL, E, k, off["bytes"], stride, [v.data_ptr() for v in views], stride,
                     slab.data_ptr(), copy_stream, 0)
    ws = smoe.workspace(dims, C)
    x = torch.empty((C, dims.d_model), dtype=torch.int16, device="cuda")
    idx = torch.empty((C, k), dtype=torch.int32, device="cuda")
    w = torch.empty((C, k), dtype=torch.float32, device="cuda")
    mu = min(E, C * k)
    uids = torch.empty(mu, dtype=torch.int32, device="cuda")
    ucount = torch.zeros(1, dtype=torch.int32, device="cuda")
    offs = torch.empty(mu + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(C * k, dtype=torch.int32, device="cuda")
    table = torch.empty(E, dtype=torch.int64, device="cuda")
    unions = []
    # per chunk-layer timing of the last timed prompt (chunk order): routing
    # (compute stream), the host side of the routed acquisition, and the span
    # of that acquisition's fills on the copy stream
    timing = {"on": False, "ev": [], "host_s": []}

    def chunk_layer(c, L):
        r = resid[c * C:(c + 1) * C]
        r.copy_(prompt[c * C:(c + 1) * C])
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if timing["on"] else None
        if ev:
            ev[0].record()
        smoe.route(dims, r, x, router[L], bias[L], idx, w, ws)
        if ev:
            ev[1].record()
            ev[2].record(copy_stream)
        t0 = time.perf_counter()
        # the library reads the routing back, forms the union in first-touch
        # order and acquires it (fills in that order), then writes the table
        unions.append(len(ring.acquire_routed(L, idx, table)))
        if ev:
            timing["host_s"].append(time.perf_counter() - t0)
            ev[3].record(copy_stream)
            timing["ev"].append(ev)
        smoe.moe_prefill_chunk(dims, x, idx, w, table, r, uids, ucount, offs, perm, ws)

    def prompt_run(tag, order):
        if order == "chunk":
            for c in range(n_chunks):
                for L in range(NL):
                    chunk_layer(c, L)
                torch.cuda.synchronize()
                log(f"{tag}: chunk {c + 1}/{n_chunks} done")
        else:
            for L in range(NL):
                for c in range(n_chunks):
                    chunk_layer(c, L)
                if L % 16 == 15 or L == NL - 1:
                    torch.cuda.synchronize()
                    log(f"{tag}: layer {L + 1}/{NL} done")

    K = args.steps
    res = {}
    for order in ("chunk", "layer"):
        for i in range(args.warmup):
            prompt_run(f"{order}-order warm-up prompt {i + 1}", order)
        s0 = ring.stats()
        n_u0 = len(unions)
        t1 = time.time()
        for i in range(K):
            timing["on"] = order == "chunk" and i == K - 1
            prompt_run(f"{order}-order timed prompt {i + 1}", order)
        timing["on"] = False
        torch.cuda.synchronize()
        dt = time.time() - t1
        s1 = ring.stats()
        hits, misses = s1["hits"] - s0["hits"], s1["misses"] - s0["misses"]
        h2d = s1["h2d_bytes"] - s0["h2d_bytes"]
        res[order] = {"tok_s": K * T / dt, "ms": dt * 1000.0 / K, "mean_union": float(np.mean(unions[n_u0:])),
                      "hit_rate": hits / max(1, hits + misses), "misses_per_prompt": misses / K,
                      "h2d_bytes_per_prompt": h2d / K, "h2d_gbps": h2d / dt / 1e9,
                      "h2d_frac_of_pinned": h2d / dt / 1e9 / link["pinned_h2d_gbps"]}
        log(f"ring prefill, {order} order: {res[order]['tok_s']:.1f} prompt tokens/s, hit rate "
            f"{res[order]['hit_rate']:.3f}, H2D {res[order]['h2d_gbps']:.1f} GB/s")
    ring.release()
    ring.destroy()
    # first-touch firing: how much a fill could start earlier if it fired as
    # soon as its first token was routed, against how long the fills take
    route_us = np.array([e[0].elapsed_time(e[1]) * 1e3 for e in timing["ev"]])
    fill_us = np.array([e[2].elapsed_time(e[3]) * 1e3 for e in timing["ev"]])
    host_us = np.array(timing["host_s"]) * 1e6
    per_cl_us = res["chunk"]["ms"] * 1e3 / (n_chunks * NL)
    with_fills = fill_us > 1.0
    f1 = {"chunk_layers": int(len(route_us)), "route_us_mean": float(route_us.mean()),
          "acquire_host_us_mean": float(host_us.mean()),
          "fill_span_us_mean_when_missing": float(fill_us[with_fills].mean()) if with_fills.any() else 0.0,
          "chunk_layers_with_fills": int(with_fills.sum()), "chunk_layer_us_mean": per_cl_us,
          "max_gain_frac_of_prompt": float(route_us.sum() / (per_cl_us * len(route_us))),
          "note": "all tokens of a chunk are routed by one batch of kernels, so firing a fill at its first "
                  "token's routing could start it at most the routing time earlier; max_gain_frac_of_prompt "
                  "is that bound over the prompt time"}
    log(f"first-touch firing bound: routing {f1['route_us_mean']:.1f} us per chunk-layer, fills "
        f"{f1['fill_span_us_mean_when_missing']:.0f} us when missing, at most "
        f"{100 * f1['max_gain_frac_of_prompt']:.2f}% of the prompt time")
    f = res["chunk"]
    out = {
        "metric": "ring-backed layer-major prefill prompt tokens/s (235B-shape, 512-token prompt, chunks of 64, "
                  f"{n_slots}-slot HBM ring over a host vault" + (")" if dims.bits == 4 else ", SMOE-Q2)"),
        "value": f["tok_s"], "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": f["ms"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"q{dims.bits}-affine codes as fp16 MFMA inputs, fp32 accumulation with the affine step folded "
                 "per chunk; float64 router",
        "data": "synthetic (Zipf(1.1) logit bias, N(0,1) bf16 prompt hidden states fed to every layer)",
        "config": {"workload": f"{wl.name}-ring{n_slots}", "layers": NL, "prompt_tokens": T, "chunk": C,
                   "ring_slots": n_slots, "parallelism": "single GPU"},
        "mean_union": f["mean_union"], "hit_rate": f["hit_rate"], "misses_per_prompt": f["misses_per_prompt"],
        "h2d_bytes_per_prompt": f["h2d_bytes_per_prompt"], "h2d_gbps": f["h2d_gbps"],
        "vault_layers_page_locked": n_pinned,
        "host_link": dict(link, h2d_frac_of_pinned=f["h2d_frac_of_pinned"]),
        "layer_outer": res["layer"],
        "first_touch_firing": f1,
    }
    del views
    for v in vault:
        v.free()
    print(json.dumps(out), flush=True)


def h2d_references(nbytes=1 << 30, reps=4):
    """Host-to-device copy rates of the ring's two vault kinds: hipMemcpyAsync
    from page-locked memory (hipHostMalloc) and from pageable memory."""
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    dev = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    pinned = smoe.PinnedHost(nbytes)
    pageable = torch.ones(nbytes, dtype=torch.uint8)
    out = {}
    s = torch.cuda.current_stream()
    for name, src in (("pinned_h2d_gbps", pinned.ptr), ("pageable_h2d_gbps", pageable.data_ptr())):
        assert hip.hipMemcpyAsync(ctypes.c_void_p(dev.data_ptr()), ctypes.c_void_p(src), nbytes, 1,
                                  ctypes.c_void_p(s.cuda_stream)) == 0
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            assert hip.hipMemcpyAsync(ctypes.c_void_p(dev.data_ptr()), ctypes.c_void_p(src), nbytes, 1,
                                      ctypes.c_void_p(s.cuda_stream)) == 0
        torch.cuda.synchronize()
        out[name] = reps * nbytes / (time.perf_counter() - t0) / 1e9
    pinned.free()
    del dev, pageable
    return out


def bench_copy(args):
    """A plain elementwise copy of a known size (1 GiB read + 1 GiB written per
    launch): the calibration that turns FETCH_SIZE / WRITE_SIZE into bytes."""
    n = 1 << 28
    torch.cuda.set_device(0)
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(args.warmup):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        torch.neg(a, out=b)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    out = {"metric": "plain copy GB/s (read + write), counter calibration", "value": 2 * 4 * n / (ms / 1e3) / 1e9,
           "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": "elementwise copy 1 GiB -> 1 GiB", "bytes_read": 4 * n, "bytes_written": 4 * n}}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", choices=["decode", "prefill", "ring", "ring-prefill", "copy"], default="decode")
    ap.add_argument("--instrument-steps", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--pinned-gib", type=float, default=56.0, help="ring workloads: page-locked vault budget")
    ap.add_argument("--spec", type=int, default=0, help="ring workload: bet on gate ranks k .. k + spec - 1")
    ap.add_argument("--layers", type=int, default=None,
                    help="prefill workload: run only the first N layers (for counter passes; the default line "
                         "runs all 94)")
    ap.add_argument("--quant", choices=["q4", "q2"], default="q4",
                    help="SMOE-Q4 blobs, or the SMOE-Q2 variant (2-bit codes)")
    ap.add_argument("--shape", choices=["235b", "30b"], default="235b",
                    help="decode workload: the Qwen3-235B-A22B-shaped stack (94 layers, d_model 4096) or the "
                         "Qwen3-30B-A3B-shaped one (48 layers, d_model 2048, 256 steps by default)")
    ap.add_argument("--prewarm", action="store_true",
                    help="ring workload: after the warm-up tokens, load the most claimed experts (idle time)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="decode workload: skip the prefill sub-object (the 512-token prompt on the same stack)")
    ap.add_argument("--prefill-steps", type=int, default=3, help="decode workload: timed prompts of the prefill "
                                                                 "sub-object")
    ap.add_argument("--chunks-in-flight", type=int, default=4,
                    help="prefill: chunks kept in flight on as many streams (a causal pipeline, one layer apart)")
    ap.add_argument("--prefill-cpu-budget", type=float, default=10.0,
                    help="seconds of oracle time for the prefill sub-object's CPU baseline")
    ap.add_argument("--prefill-eager", action="store_true",
                    help="prefill workload: time the readings as eager launches, not graph replays (for counter "
                         "runs, under which replaying the prompt's graphs is slow)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the routed-expert layer is built and measured on a single "
              "MI355X (the layer has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if args.quant == "q2" and args.workload == "copy":
        print("--quant q2 applies to the decode, ring, prefill and ring-prefill workloads", file=sys.stderr)
        sys.exit(2)
    if args.shape != "235b" and args.workload != "decode":
        print("--shape applies to the decode workload only", file=sys.stderr)
        sys.exit(2)
    defaults = {"decode": (256 if args.shape == "30b" else 64, 8), "prefill": (3, 1), "ring": (256, 8), "ring-prefill": (1, 1),
                "copy": (10, 2)}[args.workload]
    args.steps = defaults[0] if args.steps is None else args.steps
    args.warmup = defaults[1] if args.warmup is None else args.warmup
    {"decode": bench_decode, "prefill": bench_prefill, "ring": bench_ring, "ring-prefill": bench_ring_prefill,
     "copy": bench_copy}[args.workload](args)


if __name__ == "__main__":
    main()
