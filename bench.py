"""Benchmark: MoE decode tokens/s and achieved HBM GB/s on Q4 expert bytes,
Qwen3-235B-A22B-shaped synthetic stack (94 MoE layers, d_model 4096, expert
ffn 1536, 128 experts, top-8, Q4 chunks of 64), batch 1, all experts resident
in HBM.

A step is one decode token through all 94 layers: exact routing (RMSNorm,
float64 gate matvec, top-8, norm_topk_prob) and the fused SMOE-Q4 expert FFN
added into the residual, each step starting from a fresh N(0,1) bf16 hidden
state.  The token's 282 kernels are captured once into a HIP graph and
replayed; the step's input copy runs eagerly inside the timed region.

Prints one JSON line.  ``--gpus N`` with N > 1 is refused: this build runs on
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


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles (the library records them on its own stream)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p(0)
            assert self.hip.hipEventCreate(ctypes.byref(h)) == 0
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
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"1 decode token through the first {n} of {wl.n_layers} layers, float64 numpy oracle, "
                      f"{spent:.1f} s of oracle time; tokens/s extrapolated to all {wl.n_layers} layers"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--instrument-steps", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the routed-expert layer is built and measured on a single "
              "MI355X (no multi-GPU path exists in this build)", file=sys.stderr)
        sys.exit(2)

    wl = synth.CONFIGS[2]
    dims = wl.dims
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

    # per-kernel timing of the gate/up kernel (the dominant kernel), eager pass
    off = synth.blob_sections(dims)
    gate_up_bytes = (off["down_codes"] - off["gate_codes"]) + (off["down_params"] - off["gate_params"])
    per_launch = dims.top_k * gate_up_bytes
    ev = HipEvents(2 * wl.n_layers)
    durs = []
    for i in range(args.instrument_steps):
        resid.copy_(H[W + i % K])
        smoe.decode_layers(dims, wl.n_layers, resid, stack.router, None, stack.tables, ws, events=ev.ev)
        torch.cuda.synchronize()
        durs += [ev.elapsed_ms(2 * L, 2 * L + 1) for L in range(wl.n_layers)]
    ev.close()
    gu_ms = float(np.mean(durs))
    achieved = per_launch / (gu_ms / 1000.0) / 1e9
    log(f"gate/up kernel: {gu_ms * 1000:.2f} us avg over {len(durs)} launches, {achieved:.0f} GB/s")

    bytes_per_token = wl.n_layers * (dims.top_k * off["bytes"] + dims.n_experts * dims.d_model * 2)
    out = {
        "metric": "MoE decode tokens/s + achieved HBM GB/s on Q4 expert bytes (235B-shape)",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4-affine weights, f16 dot products with fp32 accumulation; float64 router",
        "data": "synthetic (seeded SplitMix64 codes/scales, N(0,0.02) router, N(0,1) bf16 hidden states)",
        "config": {"workload": wl.name, "layers": wl.n_layers, "d_model": dims.d_model, "d_ff": dims.d_ff,
                   "experts": dims.n_experts, "top_k": dims.top_k, "chunk": dims.chunk, "batch": 1,
                   "vault_bytes": stack.vault.numel(), "parallelism": "single GPU"},
        "gbps_q4_expert_and_router_bytes": tok_s * bytes_per_token / 1e9,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "decode_gate_up_kernel", "bytes_per_launch": per_launch,
                     "avg_launch_us": gu_ms * 1000.0},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(stack, wl, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
