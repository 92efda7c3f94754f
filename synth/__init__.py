"""Seeded synthetic input generators shared by the oracle and the GPU path.

Holds no arithmetic of the MoE layer itself: only the SplitMix64 streams, the
SMOE-Q4 / SMOE-Q2 blob encoding of generated codes and the workload definitions.
"""
from .gen import (Dims, blob_sections, pack_blob, pack_logical, expert_logical, expert_codes,
                  expert_params_bits, pack_codes, unpack_codes, router_bits, hidden_bf16, normal_vector, zipf_bias,
                  markov_hidden, bf16_bits_from_f64, bf16_bits_to_f64, stream_key, stream_words,
                  mix64, mix64_int, BLOB_ALIGN, MAT_GATE, MAT_UP, MAT_DOWN)
from .configs import CONFIGS, Q2_WORKLOADS, SEED, Workload
