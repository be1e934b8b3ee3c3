"""Pins of the oracle's RoPE: a hand-worked closed form, the complex-number
form of the rotation, norm preservation, relative-position invariance, the
identity at position 0 (CPU only)."""
import os

import numpy as np

from oracle import rope

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rope_d4_base4.txt")


def test_golden_d4_base4():
    cases = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line.startswith("in"):
                parts = line.split()
                i = parts.index("out")
                cases.append((list(map(float, parts[1:i])), list(map(float, parts[i + 1:]))))
    assert len(cases) == 2
    c, s = rope.cos_sin_table([2], 4, 4.0)
    for x, want in cases:
        got = rope.apply_rope(np.array(x, np.float32).reshape(1, 1, 4), c, s).ravel()
        assert np.allclose(got, want, atol=1e-6), (x, got, want)


def test_theta_schedule_textbook_2d():
    # D = 2: a single pair rotated by pos * base^0 = pos radians.
    for pos in (0, 1, 3, 10):
        c, s = rope.cos_sin_table([pos], 2, 10000.0)
        r = rope.apply_rope(np.array([[[1.0, 0.0]]], np.float32), c, s).ravel()
        assert np.allclose(r, [np.cos(pos), np.sin(pos)], atol=1e-6)


def test_complex_form():
    rng = np.random.default_rng(1)
    d = 64
    pos = np.array([0, 7, 12345, 598399])
    x = rng.standard_normal((len(pos), 3, d)).astype(np.float32)
    c, s = rope.cos_sin_table(pos, d, 10000.0)
    r = rope.apply_rope(x, c, s)
    theta = np.array(rope.inv_freq(d, 10000.0))
    z = x[..., : d // 2].astype(np.float64) + 1j * x[..., d // 2:].astype(np.float64)
    rot = z * np.exp(1j * pos[:, None, None] * theta[None, None, :])
    want = np.concatenate([rot.real, rot.imag], axis=-1)
    assert np.allclose(r, want, atol=2e-5)


def test_table_matches_numpy_trig():
    pos = np.arange(0, 600000, 4999)
    c, s = rope.cos_sin_table(pos, 128, 10000.0)
    ang = pos[:, None].astype(np.float64) * np.array(rope.inv_freq(128, 10000.0))[None, :]
    # a second trig implementation agrees to within one float32 rounding
    assert np.max(np.abs(c - np.cos(ang))) <= 2.0 ** -24 * 1.0001
    assert np.max(np.abs(s - np.sin(ang))) <= 2.0 ** -24 * 1.0001


def test_norm_preserved():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 4, 128)).astype(np.float32)
    pos = rng.integers(0, 600000, size=50)
    c, s = rope.cos_sin_table(pos, 128, 10000.0)
    r = rope.apply_rope(x, c, s)
    n0 = np.linalg.norm(x.astype(np.float64), axis=-1)
    n1 = np.linalg.norm(r.astype(np.float64), axis=-1)
    assert np.max(np.abs(n1 / n0 - 1)) < 1e-6


def test_position_zero_is_identity():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 2, 128)).astype(np.float32)
    c, s = rope.cos_sin_table([0], 128, 10000.0)
    assert np.array_equal(rope.apply_rope(x, c, s), x)


def test_relative_position_invariance():
    rng = np.random.default_rng(4)
    d = 128
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, d)).astype(np.float32)
    for m, n, delta in [(5, 2, 1000), (100, 4000, 250000), (0, 11967, 586432)]:
        dots = []
        for shift in (0, delta):
            cq, sq = rope.cos_sin_table([m + shift], d, 10000.0)
            ck, sk = rope.cos_sin_table([n + shift], d, 10000.0)
            a = rope.apply_rope(q, cq, sq).astype(np.float64).ravel()
            b = rope.apply_rope(k, ck, sk).astype(np.float64).ravel()
            dots.append(a @ b)
        assert abs(dots[0] - dots[1]) < 1e-4 * (np.linalg.norm(q) * np.linalg.norm(k))


def test_chunk_positions():
    p = rope.chunk_positions(8, 4, 96)
    assert p[0] == 768 and p[-1] == 768 + 4 * 96 - 1 and len(p) == 384
