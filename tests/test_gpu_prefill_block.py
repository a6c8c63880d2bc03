"""GPU parity of kvq_sdpa_prefill (MFMA) over block-quantized caches (FP8-E4M3
with an fp32 scale, MX-FP4 with an E8M0 scale, per 32 elements of a row)
against the oracle's fp64 attention on the same quantized cache, and the same
identities as the affine caches: the per-tile causal skip is bit-identical to
scanning every tile, data past kv_len cannot matter; a zero mask agrees with
no mask within the gate."""
import numpy as np
import pytest
import torch

import oracle
import quantized_kv_cache_head_amd as kvq
import quantized_kv_cache_head_amd.workloads as wl
from _gpu import DEV, check_attention, say
from test_gpu_decode import fill_caches
from test_gpu_prefill import run_prefill

pytestmark = pytest.mark.gpu

BLOCK_MODES = [kvq.FP8E4M3_B32, kvq.MXFP4_B32, kvq.MXFP8_B32, kvq.FP8E5M2_B32, kvq.INT8_B32, kvq.MXFP4E1M2_B32]


@pytest.mark.parametrize("qmode", BLOCK_MODES)
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_block_prefill_parity_shapes(qmode, D, G):
    B, Hkv, S = 2, 2, 600
    Hq = Hkv * G
    Lq, kv_len = 150, 530                         # ragged row tiles and key tiles
    say(f"block prefill qmode={qmode} D={D} G={G}")
    K, V = fill_caches(qmode, B, Hkv, S, D, 560, seed=D + G + 5)
    q = wl.to_bf16_values(np.random.default_rng(G + D + 1).standard_normal((B, Hq, Lq, D)).astype(np.float32))
    ref = oracle.sdpa(q, K[1], V[1], kv_len, causal=True)
    for od in (torch.bfloat16, torch.float32):
        check_attention(run_prefill(q, K, V, kv_len, out_dtype=od), ref, f"qmode {qmode} D {D} G {G} {od}")


@pytest.mark.parametrize("qmode", BLOCK_MODES)
@pytest.mark.parametrize("Lq,kv_len", [(1, 1), (1, 77), (33, 33), (65, 200), (257, 1000)])
def test_block_prefill_lengths(qmode, Lq, kv_len):
    B, Hkv, G, S, D = 1, 2, 2, 1024, 128
    say(f"block prefill qmode={qmode} Lq={Lq} kv_len={kv_len}")
    K, V = fill_caches(qmode, B, Hkv, S, D, kv_len, seed=Lq * 5 + kv_len)
    q = wl.to_bf16_values(np.random.default_rng(Lq + 9).standard_normal((B, Hkv * G, Lq, D)).astype(np.float32))
    ref = oracle.sdpa(q, K[1], V[1], kv_len, causal=True)
    check_attention(run_prefill(q, K, V, kv_len, out_dtype=torch.float32), ref, f"Lq {Lq} kv {kv_len}")


@pytest.mark.parametrize("qmode", BLOCK_MODES)
def test_block_prefill_fp32(qmode):
    """fp32 queries and fp32 inputs to the cache (hi + lo fp16 limbs of q)."""
    B, Hkv, G, S, D, T = 1, 2, 2, 256, 64, 64
    say(f"block prefill fp32 qmode={qmode}")
    K, V = fill_caches(qmode, B, Hkv, S, D, T, seed=71, bf16=False)
    q = np.random.default_rng(72).standard_normal((B, Hkv * G, T, D)).astype(np.float32)
    ref = oracle.sdpa(q, K[1], V[1], T, causal=True)
    check_attention(run_prefill(q, K, V, T, q_bf16=False, out_dtype=torch.float32), ref, "fp32")


@pytest.mark.parametrize("qmode", BLOCK_MODES)
def test_block_prefill_identities(qmode):
    B, Hkv, G, S, D, Lq = 1, 2, 4, 1024, 128, 200
    K, V = fill_caches(qmode, B, Hkv, S, D, 1024, seed=81)
    q = wl.to_bf16_values(np.random.default_rng(82).standard_normal((B, Hkv * G, Lq, D)).astype(np.float32))
    say(f"block prefill identities qmode={qmode}")
    for kv_len in (200, 700):
        a = run_prefill(q, K, V, kv_len)
        assert torch.equal(a, run_prefill(q, K, V, kv_len, no_skip=True))
        # a zero mask: the same within rounding (it bounds the V scales per tile)
        ref_c = oracle.sdpa(q, K[1], V[1], kv_len, causal=True)
        check_attention(run_prefill(q, K, V, kv_len, mask=np.zeros((Lq, S), np.float32)), ref_c, "zero mask")
    kv_len = 700
    base = run_prefill(q, K, V, kv_len)
    # a non-causal additive mask vs the oracle
    rng = np.random.default_rng(83)
    mask = np.where(rng.random((Lq, S)) < 0.4, -np.inf, 0.0).astype(np.float32)
    mask[:, 3] = 0.0
    ref = oracle.sdpa(q, K[1], V[1], kv_len, mask=mask, causal=False)
    check_attention(run_prefill(q, K, V, kv_len, causal=False, mask=mask, out_dtype=torch.float32), ref, "mask")
    # garbage past kv_len: random codes (FP8 NaN codes included), NaN / 0xFF scales
    for dc, _ in (K, V):
        dc.codes[:, :, kv_len:] = torch.randint(0, 256, dc.codes[:, :, kv_len:].shape, dtype=torch.uint8, device=DEV)
        if dc.scales.dtype == torch.uint8:
            dc.scales[:, :, kv_len:] = 0xFF
        else:
            dc.scales[:, :, kv_len:] = float("nan")
    assert torch.equal(base, run_prefill(q, K, V, kv_len))


def test_block_prefill_long_chunk_sampled():
    """The long-prefill shape (B 1, 32/16 heads, D 256, Lq 2048 chunk at
    kv_len 8192) over an MX-FP4 cache, in the benchmark's launch
    configuration; 64 rows x 32 heads checked against the oracle, every tile
    boundary included."""
    w = wl.LONGPREFILL
    S, kv_len, Lq = 8192, 8192, w.Lq
    say(f"block prefill long chunk MX-FP4 kv_len={kv_len}")
    K, V = fill_caches(kvq.MXFP4_B32, 1, w.Hkv, S, w.D, kv_len, seed=91, outliers=False)
    q = wl.to_bf16_values(np.random.default_rng(92).standard_normal((1, w.Hq, Lq, w.D)).astype(np.float32))
    out = run_prefill(q, K, V, kv_len)
    # first and last row of every 64-row query tile (this shape's tile height)
    rows_r = np.sort(np.concatenate([np.arange(0, Lq, 64), np.arange(63, Lq, 64)]))
    rows = np.array([(0, h, r) for h in range(w.Hq) for r in rows_r], np.int32)
    ref = oracle.sdpa(q, K[1], V[1], kv_len, causal=True, rows=rows)
    idx_h = torch.from_numpy(rows[:, 1].astype(np.int64)).to(DEV)
    idx_r = torch.from_numpy(rows[:, 2].astype(np.int64)).to(DEV)
    check_attention(out[0, idx_h, idx_r], ref, "long chunk rows")
