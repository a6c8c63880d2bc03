"""The affine scatter kernel forms scale = RN(range / (qmax - qmin)) without a
division: a product with RN(1 / n) and one fused residual step.  This CPU
test runs tests/csrc/div_const_sweep.c, which checks that formula against the
correctly rounded quotient for every finite non-negative float, for n = 255
(int8) and n = 15 (4-bit)."""
import os
import shutil
import subprocess

import pytest

SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "div_const_sweep.c")


@pytest.mark.timeout(600)
def test_scale_division_by_constant_is_exact(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "div_const_sweep")
    # contraction off: the two fmaf calls are the only fused operations
    r = subprocess.run([gcc, "-O2", "-fopenmp", "-ffp-contract=off", "-o", exe, SRC, "-lm"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    env["OMP_NUM_THREADS"] = str(min(8, os.cpu_count() or 1))
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=560)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "n=255 mismatches=0" in r.stdout and "n=15 mismatches=0" in r.stdout, r.stdout
