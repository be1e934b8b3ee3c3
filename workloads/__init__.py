"""Seeded synthetic workloads for the KV-cache upkeep + chunk-attention path.

This package holds the shapes of the five workloads and the seeded input
generators.  It is the only module that both the oracle-side tests and the
GPU-side tests and benchmark use; it contains none of the method's arithmetic
(no RoPE, no quantization, no attention): only shapes and random numbers.
"""
from .configs import WORKLOADS, Workload, get_workload
from .generate import (
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    qkv_normal,
    kv_student_t_outliers,
    out_projection_inputs,
    projection_inputs,
    query_normal,
    seed_key,
)

__all__ = [
    "WORKLOADS",
    "Workload",
    "get_workload",
    "bf16_bits_to_f32",
    "f32_to_bf16_bits",
    "qkv_normal",
    "kv_student_t_outliers",
    "out_projection_inputs",
    "projection_inputs",
    "query_normal",
    "seed_key",
]
