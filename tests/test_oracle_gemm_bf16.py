"""Pins of the oracle's projection GEMM and its bfloat16 rounding (CPU only)."""
import numpy as np
import torch

from oracle import bf16, e4m3, gemm
from tests.gemm_model import grouped_truncation_sum as _grouped_truncation_sum


def test_bf16_rounding_matches_torch_on_float32_inputs():
    # for float32 inputs torch's cast has a single rounding, so the two must agree
    rng = np.random.default_rng(21)
    x = (rng.standard_normal(200000) * 10.0 ** rng.integers(-6, 6, 200000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16.from_f64(x.astype(np.float64)), ref)


def test_bf16_rounding_single_rounding_from_float64():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 2^-8 + 2^-40 is above the tie and must round up (a float32 double
    # rounding would land on the tie and go down).
    x = np.array([1 + 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -40, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8 + 2.0 ** -40)])
    got = bf16.to_f32(bf16.from_f64(x)).astype(np.float64)
    assert list(got) == [1.0, 1 + 2.0 ** -7, 1 + 2 * 2.0 ** -7, -(1 + 2.0 ** -7)]


def test_per_tensor_quant_closed_form():
    x = np.array([[448.0, -1.0], [0.5, 3.0]], np.float32)
    codes, s = gemm.quantize_per_tensor(x)
    assert s == np.float32(1.0)
    assert codes.tolist() == [[0x7E, 0xB8], [0x30, 0x44]]


def test_gemm_identity_and_scales():
    rng = np.random.default_rng(22)
    a_codes = rng.integers(0, 0x7E, size=(8, 16)).astype(np.uint8) | (rng.integers(0, 2, (8, 16)).astype(np.uint8) << 7)
    eye = np.where(np.eye(16, dtype=bool), 0x38, 0x00).astype(np.uint8)   # 0x38 = 1.0
    out = gemm.gemm_fp64(a_codes, np.float32(0.5), eye, np.float32(0.25))
    assert np.array_equal(out, e4m3.decode(a_codes) * 0.125)


def test_gemm_brute_force_small():
    rng = np.random.default_rng(23)
    a = rng.integers(0, 256, size=(3, 5)).astype(np.uint8)
    b = rng.integers(0, 256, size=(5, 4)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x10
    b[(b & 0x7F) == 0x7F] = 0x11
    out = gemm.gemm_fp64(a, np.float32(2.0), b, np.float32(0.5))
    for i in range(3):
        for j in range(4):
            s = sum(e4m3.decode_code(a[i, k]) * e4m3.decode_code(b[k, j]) for k in range(5))
            assert out[i, j] == s


def test_fp32_accumulation_within_bound():
    rng = np.random.default_rng(24)
    x = rng.standard_normal((16, 512)).astype(np.float32)
    w = (rng.standard_normal((512, 8)) / np.sqrt(512)).astype(np.float32)
    xc, sx = gemm.quantize_per_tensor(x)
    wc, sw = gemm.quantize_per_tensor(w)
    exact = gemm.gemm_fp64(xc, sx, wc, sw)
    acc = np.zeros((16, 8), np.float32)
    a = e4m3.decode(xc).astype(np.float32)
    b = e4m3.decode(wc).astype(np.float32)
    for k in range(512):
        acc = acc + a[:, k:k + 1] * b[k:k + 1, :]     # float32, sequential
    acc = acc.astype(np.float64) * (float(sx) * float(sw))
    assert np.all(np.abs(acc - exact) <= gemm.error_bound(xc, sx, wc, sw) + 1e-30)


def test_code_exponents():
    assert gemm.code_exponents(np.array([0x38]))[0] == 0         # 1.0
    assert gemm.code_exponents(np.array([0x7E]))[0] == 8         # 448
    assert gemm.code_exponents(np.array([0x01]))[0] == -6        # 2^-9, subnormal
    assert gemm.code_exponents(np.array([0x08]))[0] == -6        # 2^-6, smallest normal
    assert np.isneginf(gemm.code_exponents(np.array([0x80]))[0])
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]
    codes = codes[(codes & 0x7F) != 0]
    v = np.abs(e4m3.decode(codes))
    e = gemm.code_exponents(codes)
    normal = ((codes >> 3) & 0xF) != 0
    assert np.all(2.0 ** e[normal] <= v[normal]) and np.all(v[normal] < 2.0 ** (e[normal] + 1))
    assert np.all(v[~normal] < 2.0 ** e[~normal])


def test_group_truncation_model_within_bound():
    """The bound covers the truncating model on full-range codes (the hardest
    case: products spread over 35 binades) and on N(0,1)-like data."""
    rng = np.random.default_rng(7)
    for trial in range(3):
        a = rng.integers(0, 256, (6, 64), dtype=np.uint8)
        b = rng.integers(0, 256, (64, 5), dtype=np.uint8)
        a[(a & 0x7F) == 0x7F] = 0x7E
        b[(b & 0x7F) == 0x7F] = 0x7E
        exact = gemm.gemm_fp64(a, 1.0, b, 1.0)
        model = _grouped_truncation_sum(a, b)
        bound = gemm.error_bound(a, 1.0, b, 1.0)
        assert np.all(np.abs(model - exact) <= bound)
        # the group term is what makes it hold: the float32-only bound is too tight
        f32_only = 64 * 2.0 ** -24 * (np.abs(e4m3.decode(a)) @ np.abs(e4m3.decode(b)))
        if trial == 0:
            assert np.any(np.abs(model - exact) > f32_only)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    w = rng.standard_normal((256, 3)).astype(np.float32)
    xc, sx = gemm.quantize_per_tensor(x)
    wc, sw = gemm.quantize_per_tensor(w)
    model = _grouped_truncation_sum(xc, wc) * (float(sx) * float(sw))
    exact = gemm.gemm_fp64(xc, sx, wc, sw)
    assert np.all(np.abs(model - exact) <= gemm.error_bound(xc, sx, wc, sw))


def test_group_truncation_model_reproduces_cancellation_cases():
    """448 + c - 448 within one group keeps c only to multiples of 2^(8-13);
    in different groups c survives whole."""
    c = np.array([0x1E], np.uint8)                      # 0.109375
    a = np.zeros((1, 16), np.uint8)
    a[0, 0], a[0, 1], a[0, 2] = 0x7E, 0xFE, c[0]
    b = np.full((16, 1), 0x38, np.uint8)
    assert _grouped_truncation_sum(a, b)[0, 0] == 0.09375
    a[0, 2], a[0, 9] = 0, c[0]
    assert _grouped_truncation_sum(a, b)[0, 0] == 0.109375


def _designed_group_losses():
    """Rows whose every group holds one product of exponent 8 (448 x 1) and
    seven just below the alignment step 2^(8-13): 0.029296875 = 2^-6 x 1.875,
    each of which the grouped truncation drops whole, and its negation."""
    small = 0x0F                                       # 2^-6 * (1 + 7/8)
    a = np.full((2, 64), small, np.uint8)
    a[:, ::8] = 0x7E                                   # 448 leads each group
    a[1] |= 0x80                                       # the negated row
    b = np.full((64, 1), 0x38, np.uint8)               # 1.0
    return a, b


def _worst_ratio(a, b, align_bits):
    exact = gemm.gemm_fp64(a, 1.0, b, 1.0)
    model = _grouped_truncation_sum(a, b)
    bound = gemm.error_bound(a, 1.0, b, 1.0, align_bits=align_bits)
    return float(np.max(np.abs(model - exact) / bound))


def test_group_term_is_tight_on_designed_losses():
    """The bound is not loose: on the designed rows the model's error reaches
    0.82 of it (7 of the 8 alignment steps of each group), and a bound built
    with a coarser alignment (align_bits <= 10) would stay under a quarter."""
    a, b = _designed_group_losses()
    r = _worst_ratio(a, b, 13)
    print(f"designed groups: error / bound = {r:.3f}")
    assert 0.25 <= r <= 1.0
    assert r > 0.8
    for bits in (10, 9, 8):
        assert _worst_ratio(a, b, bits) < 0.25, bits
    # the float32-only bound misses these losses by far
    exact = gemm.gemm_fp64(a, 1.0, b, 1.0)
    f32_only = 64 * 2.0 ** -24 * (np.abs(e4m3.decode(a)) @ np.abs(e4m3.decode(b)))
    assert np.all(np.abs(_grouped_truncation_sum(a, b) - exact) > 100 * f32_only)


def test_group_term_on_full_range_codes():
    """Random full-range codes (products over 35 binades): the model's error
    exceeds the float32-only bound on some outputs and stays within the group
    bound everywhere; its worst ratio to the bound (about 0.06: random groups
    rarely lose all eight steps, and the bound takes the group's largest
    exponents of A and B separately) is printed."""
    rng = np.random.default_rng(31)
    a = rng.integers(0, 256, (16, 128), dtype=np.uint8)
    b = rng.integers(0, 256, (128, 8), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x7E
    b[(b & 0x7F) == 0x7F] = 0x7E
    r = _worst_ratio(a, b, 13)
    print(f"full-range codes: worst error / bound = {r:.3f}")
    assert r <= 1.0
    exact = gemm.gemm_fp64(a, 1.0, b, 1.0)
    f32_only = 128 * 2.0 ** -24 * (np.abs(e4m3.decode(a)) @ np.abs(e4m3.decode(b)))
    assert np.any(np.abs(_grouped_truncation_sum(a, b) - exact) > f32_only)
