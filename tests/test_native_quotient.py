"""The per-row reciprocal quotient the quantize kernels use is exact.

The kernels replace the per-element IEEE division fl32(x*127)/s by a
reciprocal computed once per row plus one fused correction step, and round
with an fp32 add of +-0.5 and a truncating conversion (see
tests/native/quotient_check.c).  This test compiles that C program with gcc
and runs it: it walks every fp16 pair (x, s) with |x| <= s, and every
product of a code in [-127, 127] with an fp16 scale divided by 127, and
fails on any result that differs from IEEE division.  Host only.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_reciprocal_quotient_is_exact(tmp_path):
    exe = str(tmp_path / "quotient_check")
    src = os.path.join(HERE, "native", "quotient_check.c")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe, src, "-lm"], check=True)
    p = subprocess.run([exe], stdout=subprocess.PIPE, text=True, timeout=600)
    print(p.stdout)
    assert p.returncode == 0, p.stdout
    assert "quotient_mismatch 0 code_mismatch 0 round_mismatch 0" in p.stdout
    assert "dequant_mismatch 0" in p.stdout
