"""Projection step of the largest workload: per-tensor FP8 quantization and an
FP8 GEMM with float32-or-better accumulation.

The pages name a fused FP8 matmul in the serving step (page "Runway explains how
it serves a 57B video model in real time", fourth paragraph) and matmul tuning
(page "Runway partage la construction de Runway Characters", third paragraph)
without a formula.  Reading taken:

    s_x = f32(amax(X) / 448),  Xq = e4m3.encode(f32(X / s_x))     (per tensor)
    s_w = f32(amax(W) / 448),  Wq = e4m3.encode(f32(W / s_w))
    QKV = bf16( s_x * s_w * sum_k decode(Xq[m,k]) * decode(Wq[k,n]) )

with the sum and the product of the scales taken in float64 and one rounding
to bfloat16 (nearest, ties to even) at the end.
"""
from __future__ import annotations

import numpy as np

from . import bf16, e4m3, quant


def quantize_per_tensor(x_f32: np.ndarray):
    """(codes uint8 same shape, scale float32) with one scale for the whole tensor."""
    x = np.asarray(x_f32, dtype=np.float32)
    codes, scale = quant.quantize_rows(x.reshape(1, -1))
    return codes.reshape(x.shape), np.float32(scale[0])


def gemm_fp64(a_codes, s_a, b_codes, s_b) -> np.ndarray:
    """float64 value of s_a * s_b * decode(A) @ decode(B)."""
    a = e4m3.decode(a_codes)
    b = e4m3.decode(b_codes)
    return (float(s_a) * float(s_b)) * (a @ b)


def gemm_bf16(a_codes, s_a, b_codes, s_b) -> np.ndarray:
    """The GEMM rounded once to bfloat16 (bit patterns)."""
    return bf16.from_f64(gemm_fp64(a_codes, s_a, b_codes, s_b))


def error_bound(a_codes, s_a, b_codes, s_b) -> np.ndarray:
    """Bound on |fp32-accumulated result - exact| before the bf16 rounding:
    K * 2^-24 * s_a*s_b * sum_k |a||b| (float32 accumulation of exact products)."""
    a = np.abs(e4m3.decode(a_codes))
    b = np.abs(e4m3.decode(b_codes))
    k = a.shape[1]
    return k * 2.0 ** -24 * (float(s_a) * float(s_b)) * (a @ b)
