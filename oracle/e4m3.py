"""OCP FP8 E4M3FN codec, written from the format's definition.

The pages say only that the cache is stored in FP8 (page "Runway explains how
it serves a 57B video model in real time", fourth paragraph).  The format
taken is OCP E4M3FN: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
no infinities, a single NaN magnitude (0x7F / 0xFF), largest finite value 448.

decode(code):  exponent field 0 -> m * 2^-9 (subnormal); otherwise
               (1 + m/8) * 2^(e-7); 0x7F / 0xFF -> NaN.
encode(y):     the finite e4m3 value nearest to y; on a tie, the code whose
               mantissa LSB is 0; |y| >= 448 -> +-448 (saturating); the sign is
               kept when y rounds to zero.

The encoder searches the sorted table of the 127 non-negative finite values,
so it is a direct transcription of "nearest representable value".
"""
from __future__ import annotations

import numpy as np

MAX_FINITE = 448.0
NAN_CODES = (0x7F, 0xFF)


def decode_code(code: int) -> float:
    """Value of one code (Python float, exact)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# table of the 127 non-negative finite values, indexed by code 0x00..0x7E
POS_VALUES = np.array([decode_code(c) for c in range(0x7F)], dtype=np.float64)
DECODE_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)
assert np.all(np.diff(POS_VALUES) > 0), "e4m3 magnitudes must increase with the code"


def decode(codes: np.ndarray) -> np.ndarray:
    """Decode an array of uint8 codes to float64 (NaN for 0x7F / 0xFF)."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(y: np.ndarray) -> np.ndarray:
    """Encode float32 values to e4m3 codes (nearest, ties to even, saturating).

    NaN inputs are outside the definition and are rejected.
    """
    y = np.asarray(y, dtype=np.float32)
    if np.isnan(y).any():
        raise ValueError("e4m3 encode: NaN input is outside the definition")
    a = np.abs(y).astype(np.float64)
    sign = np.signbit(y).astype(np.uint8) << 7
    # index of the largest table value <= a (clamped to the table)
    lo = np.searchsorted(POS_VALUES, a, side="right") - 1
    lo = np.clip(lo, 0, len(POS_VALUES) - 1)
    hi = np.minimum(lo + 1, len(POS_VALUES) - 1)
    d_lo = a - POS_VALUES[lo]          # exact in float64 (see module docstring)
    d_hi = POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (lo % 2 == 1))
    mag = np.where(pick_hi & (hi != lo), hi, lo)
    mag = np.where(a >= MAX_FINITE, len(POS_VALUES) - 1, mag)
    return (mag.astype(np.uint8) | sign).astype(np.uint8)
