"""Pins of the oracle's quantization and attention (CPU only): closed forms,
exact brute force, error bounds, the special cases softmax attention reduces to."""
import math
from fractions import Fraction

import numpy as np

from oracle import attention, e4m3, quant


# ---------------------------------------------------------------- quantization
def test_scale_closed_form():
    x = np.zeros((3, 8), np.float32)
    x[0, 3] = 448.0
    x[0, 1] = 1.0
    x[1, 0] = -224.0
    x[1, 5] = 3.0
    x[2, :] = 7.0
    codes, scales = quant.quantize_rows(x)
    assert scales[0] == np.float32(1.0) and scales[1] == np.float32(0.5)
    assert scales[2] == np.float32(7.0) / np.float32(448.0)
    assert codes[0, 3] == 0x7E and codes[0, 1] == 0x38 and codes[0, 0] == 0x00
    assert codes[1, 0] == 0xFE and codes[1, 5] == (9 << 3) | 4  # 6.0 = 1.5 * 2^2: exponent field 2+7
    assert np.all(codes[2] == 0x7E)


def test_zero_rows_give_zero_scale_and_signed_zero_codes():
    x = np.zeros((2, 6), np.float32)
    x[1, 2] = -0.0
    codes, scales = quant.quantize_rows(x)
    assert np.all(scales == 0)
    assert codes[1, 2] == 0x80 and codes[0, 2] == 0x00
    assert np.all(quant.dequantize_rows(codes, scales) == 0)


def test_brute_force_rows_exact_rationals():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((6, 16)) * np.array([1, 10, 0.01, 300, 1e-3, 5])[:, None]).astype(np.float32)
    codes, scales = quant.quantize_rows(x)
    for r in range(x.shape[0]):
        amax = max(abs(float(v)) for v in x[r])
        s = np.float32(np.float32(amax) / np.float32(448.0))
        assert scales[r] == s
        for d in range(x.shape[1]):
            y = np.float32(x[r, d] / s)          # float32 division, correctly rounded
            a = Fraction(abs(float(y)))
            best = min(range(0x7F), key=lambda c: (abs(a - Fraction(e4m3.decode_code(c))), c % 2))
            if abs(float(y)) >= 448:
                best = 0x7E
            want = best | (0x80 if np.signbit(y) else 0)
            assert codes[r, d] == want


def test_dequantization_error_bound():
    rng = np.random.default_rng(12)
    x = rng.standard_t(3, size=(2000, 128)).astype(np.float32)
    codes, scales = quant.quantize_rows(x)
    deq = quant.dequantize_rows(codes, scales)
    a = np.abs(x.astype(np.float64))
    y = a / scales[:, None].astype(np.float64)
    normal = y >= 2.0 ** -6
    err = np.abs(deq - x)
    assert np.all(err[normal] <= 2.0 ** -4 * a[normal] * (1 + 2.0 ** -20))
    sub = ~normal
    bound = (2.0 ** -10 * scales[:, None].astype(np.float64)) * (1 + 2.0 ** -20)
    assert np.all(err[sub] <= np.broadcast_to(bound, err.shape)[sub])
    # the largest element of every row maps to +-448 exactly or one code below
    top = np.take_along_axis(codes, np.argmax(a, axis=1)[:, None], axis=1).ravel() & 0x7F
    assert np.all(top >= 0x7D)


# ---------------------------------------------------------------- attention
def _brute(q, k, v):
    d = len(q)
    s = [sum(float(q[i]) * float(kk[i]) for i in range(d)) / math.sqrt(d) for kk in k]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    z = sum(e)
    return [sum(e[j] * float(v[j][i]) for j in range(len(k))) / z for i in range(v.shape[1])]


def test_attention_brute_force():
    rng = np.random.default_rng(13)
    q = rng.standard_normal((5, 8))
    k = rng.standard_normal((9, 8)) * 2
    v = rng.standard_normal((9, 8))
    got = attention.attend_rows(q, k, v)
    for i in range(5):
        assert np.allclose(got[i], _brute(q[i], k, v), rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(14)
    d = 16
    v = rng.standard_normal((7, d))
    q = rng.standard_normal((3, d))
    # one key: output is that value
    assert np.allclose(attention.attend_rows(q, v[:1] * 3, v[:1]), np.repeat(v[:1], 3, 0))
    # identical keys: mean of the values
    k_same = np.repeat(rng.standard_normal((1, d)), 7, 0)
    assert np.allclose(attention.attend_rows(q, k_same, v), np.repeat(v.mean(0, keepdims=True), 3, 0))
    # zero query: uniform weights
    assert np.allclose(attention.attend_rows(np.zeros((1, d)), rng.standard_normal((7, d)), v),
                       v.mean(0, keepdims=True))
    # a dominant score selects its row
    k = rng.standard_normal((7, d)) * 0.01
    k[4] = q[0] * 1000
    assert np.allclose(attention.attend_rows(q[:1], k, v), v[4:5], atol=1e-9)


def test_grouped_query_heads():
    rng = np.random.default_rng(15)
    q = rng.standard_normal((4, 4, 8))
    k = rng.standard_normal((6, 2, 8))
    v = rng.standard_normal((6, 2, 8))
    out = attention.attend(q, k, v)
    for h in range(4):
        kv = h // 2
        assert np.allclose(out[:, h], attention.attend_rows(q[:, h], k[:, kv], v[:, kv]))
    sub = attention.attend(q, k, v, rows=[3, 1])
    assert np.allclose(sub, out[[3, 1]])
