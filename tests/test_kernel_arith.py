"""Exhaustive CPU checks of arithmetic identities the kernels rely on (no GPU involved).

* kernel 1's INT4 group scale: the fp32 quotient a / 7, formed as a * fp32(1/7) plus one
  fma correction with the exact residual, is the correctly rounded quotient for every
  non-negative finite fp32 a (the scale's definition, s = fp16(fp32(a / 7)), in the
  review's section 3 quantizer).  The C check runs all 2^31 - 2^23 values.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_fma_corrected_division_by_7_is_correctly_rounded(tmp_path):
    exe = str(tmp_path / "div7")
    r = subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe, os.path.join(HERE, "arith", "div7.c"), "-lm"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and "0 mismatches" in r.stdout, r.stdout[-2000:]
