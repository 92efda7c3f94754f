"""Writes the stored expected values under tests/golden/ from the CPU oracle.

Calls only ``synth`` (inputs) and ``oracle`` (expected values).  Run from the
repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402


def tiny_decode():
    wl = synth.CONFIGS[0]
    dims = wl.dims
    experts = {e: synth.expert_logical(wl.seed, dims, 0, e) for e in range(dims.n_experts)}
    wr = synth.router_bits(wl.seed, dims, 0)
    r = synth.hidden_bf16(wl.seed, 0, dims.d_model).astype(np.float64)
    out = oracle.moe_layer(r, wr, experts, dims)
    return {
        "workload": wl.name,
        "what": "one decode token through one MoE layer: x bits, routed experts, mixing weights, MoE output",
        "seed": wl.seed,
        "x_bits": [int(b) for b in out["x_bits"]],
        "idx": [int(e) for e in out["idx"]],
        "w": [float(v) for v in out["w"]],
        "y": [float(v) for v in out["y"]],
    }


def main():
    with open(os.path.join(HERE, "tiny_decode.json"), "w") as f:
        json.dump(tiny_decode(), f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
