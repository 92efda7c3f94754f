"""The five synthetic workloads (shapes, distributions, step counts).

Shapes are the MoE-layer geometry of the two models the pages run: a
Qwen3-30B-A3B-shaped stack (48 MoE layers, d_model 2048, expert ffn 768) and a
Qwen3-235B-A22B-shaped stack (94 MoE layers, d_model 4096, expert ffn 1536);
both have 128 experts with top-8 routing and norm_topk_prob (System Overview,
"What Happens at Each Generated Token Step"; Optimizations, "Routing Is
Exact").  Prefill chunks hold up to 64 tokens (Optimizations, "Prefill Reads
Each Expert Once").  Seed 1337 is the pages' canonical-benchmark seed
(Optimizations, header).
"""
from __future__ import annotations

from dataclasses import dataclass, field

from .gen import Dims

SEED = 1337


@dataclass
class Workload:
    name: str
    dims: Dims
    n_layers: int
    steps: int                 # decode tokens, or prompt tokens for prefill
    mode: str                  # "decode", "prefill", "ring"
    prefill_chunk: int = 64
    zipf_s: float = 0.0        # > 0: per-expert Zipf logit bias
    ring_slots: int = 0
    markov: tuple = ()         # (keep, fresh) for Markov hidden states
    seed: int = SEED
    notes: str = field(default="")


TINY = Workload(
    name="tiny-decode-1layer-d256-f128-e16-k4",
    dims=Dims(256, 128, 16, 4, 32),
    n_layers=1, steps=1, mode="decode")

QWEN30B_DECODE = Workload(
    name="qwen3-30b-a3b-shape-decode-48L-d2048-f768-e128-k8-q4c64",
    dims=Dims(2048, 768, 128, 8, 64),
    n_layers=48, steps=256, mode="decode")

QWEN235B_DECODE = Workload(
    name="qwen3-235b-a22b-shape-decode-94L-d4096-f1536-e128-k8-q4c64",
    dims=Dims(4096, 1536, 128, 8, 64),
    n_layers=94, steps=64, mode="decode")

QWEN235B_PREFILL = Workload(
    name="qwen3-235b-a22b-shape-prefill-512tok-chunk64-94L-zipf1.1",
    dims=Dims(4096, 1536, 128, 8, 64),
    n_layers=94, steps=512, mode="prefill", prefill_chunk=64, zipf_s=1.1)

QWEN235B_RING = Workload(
    name="qwen3-235b-a22b-shape-ring-decode-256tok-1536slots-markov0.7",
    dims=Dims(4096, 1536, 128, 8, 64),
    n_layers=94, steps=256, mode="ring", ring_slots=1536, markov=(0.7, 0.3))

CONFIGS = [TINY, QWEN30B_DECODE, QWEN235B_DECODE, QWEN235B_PREFILL, QWEN235B_RING]

# SMOE-Q2 variants ("Q2 Vaults -- the Next 2x, Twice Over", Optimizations page:
# a 2-bit vault halves every blob and doubles the ring's slots).  Same shapes,
# seeds and distributions as the Q4 workloads; the ring keeps the Q4 ring's HBM
# budget (1536 Q4 slots = 16.31 GB), which holds 2764 Q2 blobs.
QWEN235B_DECODE_Q2 = Workload(
    name="qwen3-235b-a22b-shape-decode-94L-d4096-f1536-e128-k8-q2c64",
    dims=Dims(4096, 1536, 128, 8, 64, bits=2),
    n_layers=94, steps=64, mode="decode")

QWEN235B_RING_Q2 = Workload(
    name="qwen3-235b-a22b-shape-ring-decode-256tok-2764slots-markov0.7-q2c64",
    dims=Dims(4096, 1536, 128, 8, 64, bits=2),
    n_layers=94, steps=256, mode="ring", ring_slots=2764, markov=(0.7, 0.3))

QWEN30B_DECODE_Q2 = Workload(
    name="qwen3-30b-a3b-shape-decode-48L-d2048-f768-e128-k8-q2c64",
    dims=Dims(2048, 768, 128, 8, 64, bits=2),
    n_layers=48, steps=256, mode="decode")

QWEN235B_PREFILL_Q2 = Workload(
    name="qwen3-235b-a22b-shape-prefill-512tok-chunk64-94L-zipf1.1-q2c64",
    dims=Dims(4096, 1536, 128, 8, 64, bits=2),
    n_layers=94, steps=512, mode="prefill", prefill_chunk=64, zipf_s=1.1)

Q2_WORKLOADS = [QWEN235B_DECODE_Q2, QWEN235B_RING_Q2, QWEN30B_DECODE_Q2, QWEN235B_PREFILL_Q2]
