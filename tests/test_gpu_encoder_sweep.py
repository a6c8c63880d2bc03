"""The block quant-scatter's element encoders (magnitude clamp + gfx950
conversion instruction) against bit-level round-to-nearest-even encoders for
FP8 E4M3FN, FP8 E5M2 and FP4 E2M1 on every fp32 bit pattern
(tests/csrc/encoder_sweep.hip, built by __graft_entry__.build()).  Together
with the oracle comparison of every code and rounding tie through the C-ABI
(test_gpu_quant_scatter.py), this covers inputs no random test reaches."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "encoder_sweep")


def test_encoders_match_on_all_fp32_inputs():
    assert os.path.exists(EXE), "tests/csrc/encoder_sweep is not built: run __graft_entry__.build()"
    print("encoder sweep over 2^32 inputs", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    for fmt in ("e4m3fn", "e5m2", "e2m1"):
        assert f"{fmt}: no error, mismatches 0" in r.stdout
