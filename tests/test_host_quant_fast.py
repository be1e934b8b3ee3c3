"""Host check of the short form of the per-row quantization in the kernels.

The append and the fused projection quantize a row with a normal scale
(amax >= 448 * 2^-100) by a shorter sequence than the general one: the scale
as a corrected product with RN(1/448) and the quotient x / scale on the signed
value (device_common.hpp: scale448, div_signed).  Their results must equal the
correctly rounded float32 divisions that the oracle performs.  The C program
restates those float operations and checks the scale for every float amax of
the range and the quotient on 2^26 sampled (x, amax) pairs, signed zeros
included.  (The GPU parity tests compare the kernels' codes with the oracle's
bit for bit, rows of every form included.)
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
BUILD = os.path.join(os.path.dirname(HERE), "_build", "tests")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_short_form_of_the_row_quantization_is_exact():
    os.makedirs(BUILD, exist_ok=True)
    exe = os.path.join(BUILD, "quant_fast_check")
    src = os.path.join(HERE, "host_c", "quant_fast_check.c")
    subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-fopenmp", src, "-o", exe, "-lm"], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=600).stdout
    lines = dict(l.rsplit(" ", 1) for l in out.strip().splitlines())
    assert lines == {"scale448 mismatches": "0", "div_signed mismatches": "0"}, out
