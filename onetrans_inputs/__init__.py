"""Seeded synthetic workloads for the OneTrans block forward (data only)."""
from .workloads import (ALL, CANDIDATE_HEAVY_FP8, ONETRANS_L, ONETRANS_S, PREFILL_BATCH, TINY,
                        Workload, pyramid_schedule)
from .generate import (bf16_round, e4m3_quantize, make_append_tokens, make_ns_tokens,
                       make_s_tokens, make_weights)

__all__ = [
    "ALL", "CANDIDATE_HEAVY_FP8", "ONETRANS_L", "ONETRANS_S", "PREFILL_BATCH", "TINY", "Workload",
    "pyramid_schedule", "bf16_round", "e4m3_quantize", "make_append_tokens", "make_ns_tokens",
    "make_s_tokens", "make_weights",
]
