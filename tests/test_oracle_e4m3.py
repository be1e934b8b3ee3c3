"""Pins of the oracle's e4m3 codec against the format definition, torch's CPU
float8 cast, exact brute force and closed forms (CPU only)."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_values.txt")


def _golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                c, v = line.split()
                rows.append((int(c, 16), float(v)))
    return rows


def test_golden_values():
    for code, value in _golden():
        got = e4m3.decode_code(code)
        if np.isnan(value):
            assert np.isnan(got), hex(code)
        else:
            assert got == value and np.signbit(got) == np.signbit(value), hex(code)


def test_decode_matches_torch_for_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3.decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(ours[~nan]))


def test_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in e4m3.NAN_CODES], dtype=np.uint8)
    vals = e4m3.decode(codes).astype(np.float32)
    assert np.array_equal(e4m3.encode(vals), codes)


def test_midpoints_round_to_even_code():
    for sign in (1.0, -1.0):
        for c in range(0x7E):
            a, b = e4m3.POS_VALUES[c], e4m3.POS_VALUES[c + 1]
            mid = np.float32((a + b) / 2)          # exact: at most 5 significant bits
            assert float(mid) == (a + b) / 2
            even = c if c % 2 == 0 else c + 1
            want = even | (0x80 if sign < 0 else 0)
            assert e4m3.encode(np.array([sign * mid], dtype=np.float32))[0] == want
            # one float32 ulp either side of the midpoint decides by distance
            below = np.nextafter(mid, np.float32(0))
            above = np.nextafter(mid, np.float32(np.inf))
            assert e4m3.encode(np.array([sign * below], np.float32))[0] == (c | (want & 0x80))
            assert e4m3.encode(np.array([sign * above], np.float32))[0] == ((c + 1) | (want & 0x80))


def test_saturation_and_signed_zero():
    big = np.array([448, 448.0001, 463.99, 464, 500, 1e30, 3.4e38], dtype=np.float32)
    assert np.all(e4m3.encode(big) == 0x7E)
    assert np.all(e4m3.encode(-big) == 0xFE)
    tiny = np.array([0.0, 1e-30, 2.0 ** -10, 2.0 ** -149], dtype=np.float32)
    assert np.all(e4m3.encode(tiny) == 0x00)
    assert np.all(e4m3.encode(-tiny) == 0x80)
    # just above half of the smallest subnormal rounds up to it
    assert e4m3.encode(np.array([np.nextafter(np.float32(2.0 ** -10), np.float32(1))]))[0] == 0x01
    with pytest.raises(ValueError):
        e4m3.encode(np.array([np.nan], dtype=np.float32))


def _nearest_exact(y: float) -> int:
    """Brute force with exact rationals: nearest finite code, ties to even, saturate."""
    a = Fraction(abs(y))
    best = None
    for c in range(0x7F):
        d = abs(a - Fraction(e4m3.decode_code(c)))
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    code = best[1]
    if abs(y) >= 448:
        code = 0x7E
    return code | (0x80 if np.signbit(np.float32(y)) else 0)


def test_brute_force_exact_rationals():
    rng = np.random.default_rng(5)
    ys = np.concatenate([
        rng.standard_normal(300).astype(np.float32) * np.float32(50),
        (rng.random(200).astype(np.float32) * np.float32(0.03)),
        -rng.random(100).astype(np.float32) * np.float32(500),
    ]).astype(np.float32)
    got = e4m3.encode(ys)
    for y, g in zip(ys, got):
        assert g == _nearest_exact(float(y)), (float(y), hex(g))


def test_matches_torch_cast_on_dense_sweep():
    # torch's CPU cast is round-to-nearest-even but not saturating (>= 464 -> NaN),
    # so the two agree on every float32 of magnitude below 464.
    top = np.array([464.0], dtype=np.float32).view(np.uint32)[0]
    bits = np.arange(0, top, 97, dtype=np.uint32)
    # plus every float32 within 40 ulps of each midpoint between adjacent codes
    mids = ((e4m3.POS_VALUES[:-1] + e4m3.POS_VALUES[1:]) / 2).astype(np.float32).view(np.uint32)
    near = (mids[:, None].astype(np.int64) + np.arange(-40, 41)[None, :]).ravel()
    bits = np.concatenate([bits, near.astype(np.uint32)])
    y = bits.view(np.float32)
    y = np.concatenate([y, -y])
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = e4m3.encode(y)
    bad = np.nonzero(ref != ours)[0]
    assert bad.size == 0, [(float(y[i]), hex(ref[i]), hex(ours[i])) for i in bad[:5]]


def test_relative_error_bound():
    rng = np.random.default_rng(7)
    y = (rng.standard_normal(200000) * 30).astype(np.float32)
    d = e4m3.decode(e4m3.encode(y))
    a = np.abs(y.astype(np.float64))
    normal = (a >= 2.0 ** -6) & (a <= 448)
    assert np.all(np.abs(d[normal] - y[normal]) <= 2.0 ** -4 * a[normal])
    sub = a < 2.0 ** -6
    assert np.all(np.abs(d[sub] - y[sub]) <= 2.0 ** -10)
