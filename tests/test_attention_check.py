"""The attention checker has teeth (CPU only): on a 47872-key N(0,1) window the
oracle's own output passes, its bf16 rounding passes, while the same output
scaled by 0.7 (30 % wrong) fails although it stays inside the absolute bounds
of the contract, and an all-zero output fails."""
import numpy as np

from oracle import attention, quant
from tests.attention_check import MAX_ABS, MEAN_ABS, attention_ok, attention_report


def _window_case(n_keys=47872, n_rows=64, d=128, seed=5):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((n_keys, d)).astype(np.float32)
    v = rng.standard_normal((n_keys, d)).astype(np.float32)
    kc, ks = quant.quantize_rows(k)
    vc, vs = quant.quantize_rows(v)
    q = rng.standard_normal((n_rows, d)).astype(np.float32)
    return attention.attend_rows(q, quant.dequantize_rows(kc, ks), quant.dequantize_rows(vc, vs))


def test_exact_output_passes():
    want = _window_case()
    assert attention_ok(attention_report(want, want))


def test_scaled_output_fails_although_inside_the_absolute_bounds():
    want = _window_case()
    wrong = 0.7 * want
    r = attention_report(wrong, want)
    # the contract's absolute bounds alone would accept it
    assert r["max"] <= MAX_ABS and r["mean"] <= MEAN_ABS
    assert not attention_ok(r)


def test_zero_output_fails():
    want = _window_case()
    assert not attention_ok(attention_report(np.zeros_like(want), want))


def test_small_rounding_passes():
    want = _window_case()
    # bf16 rounding of the output: well inside every bound
    b = want.astype(np.float32).view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    got = b.astype(np.uint32).view(np.float32)
    assert attention_ok(attention_report(got, want))
