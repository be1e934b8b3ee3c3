"""Per-(token, head) FP8 quantization of cache rows.

The pages state that the cache holds FP8 values written once at cache entry
(page "Runway explains how it serves a 57B video model in real time", fourth
paragraph) and give neither the granularity nor the scale rule.  Reading taken:
one float32 scale per (token, head) row of D values,

    amax  = max_d |x_d|
    scale = f32(amax / 448)            (correctly rounded float32 division)
    y_d   = f32(x_d / scale)           (correctly rounded float32 division)
    code  = e4m3.encode(y_d)

and when scale == 0 (all-zero row, or amax so small that amax/448 rounds to
zero) the codes are signed zeros: 0x00 for +0, 0x80 for -0 and for negative x.
The dequantized value of a code is decode(code) * scale (float64).
"""
from __future__ import annotations

import numpy as np

from . import e4m3

FP8_MAX = np.float32(448.0)


def quantize_rows(x: np.ndarray):
    """Quantize float32 rows along the last axis.

    Returns (codes uint8 same shape, scales float32 shape[:-1]).
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.divide(amax, FP8_MAX, dtype=np.float32)
    safe = np.where(scale == 0, np.float32(1.0), scale).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        y = np.divide(x, safe[..., None], dtype=np.float32)
    codes = e4m3.encode(y)
    zero_rows = scale == 0
    if zero_rows.any():
        sign = (np.signbit(x).astype(np.uint8) << 7).astype(np.uint8)
        codes = np.where(zero_rows[..., None], sign, codes).astype(np.uint8)
    return codes, scale.astype(np.float32)


def dequantize_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 values decode(code) * scale."""
    return e4m3.decode(codes) * np.asarray(scales, dtype=np.float64)[..., None]
