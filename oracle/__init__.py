"""CPU float64 oracle of the routed-expert MoE layer -- test infrastructure only.

Imported by tests/, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py``; never by the library or its binding.
"""
from .oracle import (bf16_round, bf16_to_f64, rmsnorm_bf16, router_logits, select_topk, dequant,
                     silu, expert_ffn, moe_layer, expert_union, prefill_chunk, LruRing, ring_trace,
                     HIT, MISS, PREFETCH)
