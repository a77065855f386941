"""Seeded synthetic workloads for absorbed-MLA decode.

This package only draws inputs: shapes, seeds, random values, the paged
layout and the stored-format encodings (bf16 bits, e4m3 bytes plus the
per-token scale).  It holds none of the attention arithmetic, so both the
CPU oracle and the HIP path can take their inputs from here without sharing
any of the method's code.
"""
from .configs import GQLA_GROUPS, WORKLOADS, Workload, get_workload, prefill_workload, small_workload
from .generate import (
    make_append_inputs,
    make_gqa_inputs,
    make_inputs,
    make_prefill_inputs,
    f32_to_bf16_bits,
    f32_to_e4m3_bits,
    replicate_cache,
)

__all__ = [
    "GQLA_GROUPS",
    "WORKLOADS",
    "Workload",
    "get_workload",
    "small_workload",
    "prefill_workload",
    "make_inputs",
    "make_append_inputs",
    "make_gqa_inputs",
    "make_prefill_inputs",
    "f32_to_bf16_bits",
    "f32_to_e4m3_bits",
    "replicate_cache",
]
