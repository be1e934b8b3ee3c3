"""Projection step of the largest workload: per-tensor FP8 quantization and an
FP8 GEMM with float32-or-better accumulation.

The pages name a fused FP8 matmul in the serving step (page "Runway explains how
it serves a 57B video model in real time", fourth paragraph) and matmul tuning
(page "Runway partage la construction de Runway Characters", fourth paragraph)
without a formula.  Reading taken:

    s_x = f32(amax(X) / 448),  Xq = e4m3.encode(f32(X / s_x))     (per tensor)
    s_w = f32(amax(W) / 448),  Wq = e4m3.encode(f32(W / s_w))
    QKV = bf16( s_x * s_w * sum_k decode(Xq[m,k]) * decode(Wq[k,n]) )

with the sum and the product of the scales taken in float64 and one rounding
to bfloat16 (nearest, ties to even) at the end.  error_bound() gives how far a
matrix-core result may lie from that sum before its rounding.
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


def code_exponents(codes) -> np.ndarray:
    """Unbiased exponent of each e4m3 code as a float (exponent field 0, the
    subnormals, count as -6); zero codes give -inf."""
    c = np.asarray(codes, dtype=np.uint8)
    field = ((c >> 3) & 0xF).astype(np.float64)
    e = np.where(field == 0, -6.0, field - 7.0)
    return np.where((c & 0x7F) == 0, -np.inf, e)


def error_bound(a_codes, s_a, b_codes, s_b, group: int = 8, align_bits: int = 13) -> np.ndarray:
    """Bound on |matrix-core result - exact| before the bf16 rounding.

    Two terms, both in units of the unscaled product and then scaled:

    * float32 accumulation of the partial sums: K * 2^-24 * sum_k |a||b|;
    * the FP8 matrix core's in-group alignment (a reading of "fp32
      accumulate" for this hardware, measured on gfx950): products of `group`
      consecutive k are aligned to the group's largest exponent sum
      E = max(e(a_k) + e(b_k)) and truncated to multiples of 2^(E - align_bits)
      before they are added, so a group loses less than group * 2^(E - align_bits).
      With E <= max_k e(a_k) + max_k e(b_k) over the group, the sum of these over
      the groups is a matrix product of per-group powers of two.
    """
    a = np.abs(e4m3.decode(a_codes))
    b = np.abs(e4m3.decode(b_codes))
    k = a.shape[1]
    scale = float(s_a) * float(s_b)
    bound = k * 2.0 ** -24 * (a @ b)
    if k % group == 0:
        ea = code_exponents(a_codes).reshape(a.shape[0], k // group, group).max(axis=2)
        eb = code_exponents(b_codes).reshape(k // group, group, b.shape[1]).max(axis=1)
        bound = bound + group * 2.0 ** -align_bits * (np.exp2(ea) @ np.exp2(eb))
    else:   # no grouping known: every product may lose 2^-align_bits of its own size
        bound = bound + 2.0 ** -(align_bits - 2) * (a @ b)
    return scale * bound
