"""The GPU block quantizer forms its candidate scales mu / 6 and mu / 4,
mu = m / alpha, without a division instruction sequence: a reciprocal and
one fused multiply-add correction, after an exact power-of-two rescale.  This
test compiles tests/quotient_check.c (gcc, host only), which restates that
arithmetic and checks it against IEEE division: every bf16-significand pair,
a / 6 over a dense sweep of floats, and the resulting E4M3 scale bytes over
the whole float range (the quantizer's GPU parity tests check the kernels
themselves against the oracle)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_division_free_quotients_match_ieee_division(tmp_path):
    exe = str(tmp_path / "quotient_check")
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", os.path.join(HERE, "quotient_check.c"),
           "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:]
    assert "quotient check ok" in r.stdout
