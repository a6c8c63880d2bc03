"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np
import torch

import oracle
import quantized_kv_cache_head_amd as kvq

DEV = "cuda"


def say(*a):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print(*a, flush=True)
    sys.stdout.flush()


def orc_mode(qmode):
    return {kvq.INT8_TH: oracle.INT8_TH, kvq.UINT4_TH: oracle.UINT4_TH,
            kvq.FP8E4M3_B32: oracle.FP8E4M3_B32, kvq.MXFP4_B32: oracle.MXFP4_B32,
            kvq.MXFP8_B32: oracle.MXFP8_B32, kvq.FP8E5M2_B32: oracle.FP8E5M2_B32,
            kvq.INT8_B32: oracle.INT8_B32, kvq.MXFP4E1M2_B32: oracle.MXFP4E1M2_B32}[qmode]


def new_pair(qmode, B, H, S, D):
    """(device cache, oracle host cache), both sentinel-filled."""
    dc = kvq.Cache.empty(qmode, B, H, S, D).sentinel_fill()
    hc = oracle.HostCache(orc_mode(qmode), B, H, S, D)
    return dc, hc


def assert_cache_equal(dc: "kvq.Cache", hc: "oracle.HostCache", what=""):
    """Bit-exact comparison of every byte of every plane."""
    codes = dc.codes.cpu().numpy()
    scales = dc.scales.cpu().numpy()
    bad = np.argwhere(codes != hc.codes)
    assert bad.size == 0, f"{what}: {len(bad)} code bytes differ, first at {bad[:4].tolist()}"
    sb = scales.view(np.uint8) != hc.scales.view(np.uint8)
    assert not sb.any(), f"{what}: {int(sb.sum())} scale bytes differ, first at {np.argwhere(sb)[:4].tolist()}"
    if hc.zps is not None:
        z = dc.zps.cpu().numpy()
        assert np.array_equal(z, hc.zps), f"{what}: {int((z != hc.zps).sum())} zero points differ"


def dev_input(x_np, bf16):
    """Upload float32 values (already bf16-exact when bf16) in the input dtype."""
    t = torch.from_numpy(np.ascontiguousarray(x_np))
    if bf16:
        t = t.to(torch.bfloat16)
    return t.to(DEV)


def bf16_half_ulp(ref):
    """Half an ulp of bf16 at |ref| (the rounding of the output itself)."""
    a = np.abs(ref).astype(np.float64)
    a = np.maximum(a, np.finfo(np.float32).tiny)
    e = np.floor(np.log2(a))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def check_attention(got: torch.Tensor, ref: np.ndarray, what=""):
    """Attention gate: fp32 output within 2e-3 of the fp64 oracle; bf16 output
    within 2e-3 plus half a bf16 ulp of the oracle value."""
    g = got.float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref)
    tol = 2e-3 + (bf16_half_ulp(ref) if got.dtype == torch.bfloat16 else 0.0)
    worst = np.argmax(err - tol)
    assert np.all(err <= tol), (f"{what}: max err {err.max():.3e} (tol at worst {np.ravel(tol)[worst] if np.ndim(tol) else tol:.3e},"
                                f" ref {np.ravel(ref)[worst]:.4f} got {np.ravel(g)[worst]:.4f})")
    return float(err.max())
