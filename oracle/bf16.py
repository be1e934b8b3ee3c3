"""bfloat16 helpers of the oracle (bit patterns carried as uint16)."""
from __future__ import annotations

import numpy as np


def to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact: the 16 bits are the top half)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def from_f64(x: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bit patterns, one rounding: nearest, ties to even.

    Written from the definition: the two bfloat16 neighbours of x are found from
    its float32 truncation, and the nearer one is kept (the even one on a tie).
    Values are assumed finite and inside the bfloat16 range.
    """
    x = np.asarray(x, dtype=np.float64)
    # bfloat16 values are float32 values whose low 16 bits are zero; every
    # bfloat16 value is exact in float64, so the distances below are exact.
    lo_bits = (np.abs(x).astype(np.float32).view(np.uint32) & 0xFFFF0000).astype(np.uint32)
    lo = lo_bits.view(np.float32).astype(np.float64)
    # the float32 cast may round |x| up past a bfloat16 boundary: step down if so
    over = lo > np.abs(x)
    lo_bits = np.where(over, lo_bits - 0x10000, lo_bits).astype(np.uint32)
    lo = lo_bits.view(np.float32).astype(np.float64)
    hi_bits = (lo_bits + 0x10000).astype(np.uint32)
    hi = hi_bits.view(np.float32).astype(np.float64)
    a = np.abs(x)
    d_lo = a - lo
    d_hi = hi - a
    odd = ((lo_bits >> 16) & 1) == 1
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & odd)
    mag = np.where(pick_hi, hi_bits, lo_bits) >> 16
    sign = (np.signbit(x).astype(np.uint32) << 15)
    return (mag | sign).astype(np.uint16)
