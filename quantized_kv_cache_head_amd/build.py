"""Build libkvq.so (the C-ABI HIP library) in-tree with hipcc for gfx950.

    python -m quantized_kv_cache_head_amd.build

Each ``csrc/*.hip`` file is compiled to an object in ``_build/`` (in
parallel), then linked into ``quantized_kv_cache_head_amd/libkvq.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(os.path.dirname(PKG), "_build")
LIB = os.path.join(PKG, "libkvq.so")
ARCH = os.environ.get("KVQ_ARCH", "gfx950")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-fvisibility=hidden",
    # no packed fp32 ops anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]
# files whose arithmetic must be single IEEE operations (bit-exact quantization)
NO_CONTRACT = {"quant_scatter.hip"}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, extra=()) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    flags = list(COMMON) + list(extra)
    if os.path.basename(src) in NO_CONTRACT:
        flags.append("-ffp-contract=off")
    cmd = [hipcc(), *flags, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


BENCH_CSRC = os.path.join(PKG, "bench_csrc")
BENCH_LIB = os.path.join(PKG, "libkvq_bench.so")


def build_bench(verbose: bool = False) -> str:
    """libkvq_bench.so: the kernels bench.py uses to calibrate its rooflines
    (not part of the libkvq C ABI)."""
    srcs = sorted(os.path.join(BENCH_CSRC, f) for f in os.listdir(BENCH_CSRC) if f.endswith(".hip"))
    tmp = BENCH_LIB + ".tmp"
    r = subprocess.run([hipcc(), *COMMON, "-shared", "-o", tmp, *srcs], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for the bench kernels:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, BENCH_LIB)
    if verbose:
        print(f"built {BENCH_LIB}")
    return BENCH_LIB


TESTS_CSRC = os.path.join(os.path.dirname(PKG), "tests", "csrc")


def build_test_tools(verbose: bool = False) -> list:
    """Compile the device-side test programs under tests/csrc (one executable
    per .hip file, next to its source)."""
    out = []
    if not os.path.isdir(TESTS_CSRC):
        return out
    for f in sorted(os.listdir(TESTS_CSRC)):
        if not f.endswith(".hip"):
            continue
        exe = os.path.join(TESTS_CSRC, f[:-4])
        flags = [x for x in COMMON if x not in ("-fPIC", "-fvisibility=hidden")]
        r = subprocess.run([hipcc(), *flags, "-o", exe, os.path.join(TESTS_CSRC, f)], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {f}:\n{r.stdout}\n{r.stderr}")
        out.append(exe)
        if verbose:
            print(f"built {exe}")
    return out


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
    build_bench(verbose=True)
