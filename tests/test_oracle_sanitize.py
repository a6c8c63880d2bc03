"""The CPU oracle under gcc's address and undefined-behaviour sanitizers:
tests/csrc/oracle_sanitize.c drives every oracle entry point (all seven
cache modes with -1 and out-of-range slots, every encoder on edge values,
positions, masks, attention with mask / causal / kv_len) and is built
together with oracle/kvq_oracle.c; any report aborts the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _have_asan():
    gcc = shutil.which("gcc")
    if not gcc:
        return False
    r = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True)
    return r.returncode == 0 and os.path.isabs(r.stdout.strip())


@pytest.mark.skipif(not _have_asan(), reason="gcc with libasan is not available")
def test_oracle_clean_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-O1", "-g", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           os.path.join(ROOT, "tests", "csrc", "oracle_sanitize.c"), os.path.join(ROOT, "oracle", "kvq_oracle.c"),
           "-o", exe, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "oracle sanitize ok" in r.stdout, (r.stdout[-1000:], r.stderr[-3000:])
