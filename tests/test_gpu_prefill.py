"""GPU parity of kvq_sdpa_prefill (MFMA) against the oracle's fp64 attention on
the same quantized cache, and the bit-identities of the per-tile causal bound
(skipping tiles past the bound equals scanning them)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_kv_cache_head_amd as kvq
import quantized_kv_cache_head_amd.workloads as wl
from _gpu import DEV, assert_cache_equal, check_attention, dev_input, new_pair, say
from test_gpu_decode import fill_caches, wide_range_q

pytestmark = pytest.mark.gpu


def run_prefill(q_np, K, V, kv_len, q_bf16=True, causal=True, mask=None, out_dtype=None, no_skip=False, sm=None):
    q = dev_input(q_np, q_bf16)
    kl = torch.tensor([kv_len], dtype=torch.int32, device=DEV)
    m = None if mask is None else torch.from_numpy(mask).to(DEV)
    out = kvq.sdpa_prefill(q, K[0], V[0], kv_len=kl, mask=m, causal=causal, out_dtype=out_dtype,
                           no_causal_skip=no_skip, sm_scale=sm)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("qmode", [kvq.INT8_TH, kvq.UINT4_TH])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_prefill_parity_shapes(qmode, D, G):
    B, Hkv, S = 2, 2, 600
    Hq = Hkv * G
    Lq, kv_len = 150, 530                         # ragged row tiles and key tiles
    say(f"prefill qmode={qmode} D={D} G={G}")
    K, V = fill_caches(qmode, B, Hkv, S, D, 560, seed=D + G)
    q = wl.to_bf16_values(np.random.default_rng(G + D).standard_normal((B, Hq, Lq, D)).astype(np.float32))
    ref = oracle.sdpa(q, K[1], V[1], kv_len, causal=True)
    for od in (torch.bfloat16, torch.float32):
        check_attention(run_prefill(q, K, V, kv_len, out_dtype=od), ref, f"qmode {qmode} D {D} G {G} {od}")


@pytest.mark.parametrize("Lq,kv_len", [(1, 1), (1, 77), (64, 64), (65, 200), (128, 128), (257, 1000)])
def test_prefill_lengths(Lq, kv_len):
    B, Hkv, G, S, D = 1, 2, 2, 1024, 128
    say(f"prefill Lq={Lq} kv_len={kv_len}")
    K, V = fill_caches(kvq.UINT4_TH, B, Hkv, S, D, kv_len, seed=Lq * 3 + kv_len)
    q = wl.to_bf16_values(np.random.default_rng(Lq).standard_normal((B, Hkv * G, Lq, D)).astype(np.float32))
    ref = oracle.sdpa(q, K[1], V[1], kv_len, causal=True)
    check_attention(run_prefill(q, K, V, kv_len, out_dtype=torch.float32), ref, f"Lq {Lq} kv {kv_len}")


def test_prefill_fp32_tiny_workload_shape():
    """fp32 Q/K/V, D 64, GQA 2, 64-row chunk (hi + lo fp16 limbs, fp32 output)."""
    B, Hkv, G, S, D, T = 1, 2, 2, 256, 64, 64
    say("prefill fp32")
    K, V = fill_caches(kvq.INT8_TH, B, Hkv, S, D, T, seed=31, bf16=False, outliers=False)
    q = np.random.default_rng(32).standard_normal((B, Hkv * G, T, D)).astype(np.float32)
    ref = oracle.sdpa(q, K[1], V[1], T, causal=True)
    check_attention(run_prefill(q, K, V, T, q_bf16=False, out_dtype=torch.float32), ref, "fp32")


def test_prefill_causal_skip_is_bit_identical():
    B, Hkv, G, S, D = 1, 2, 2, 2048, 256
    K, V = fill_caches(kvq.UINT4_TH, B, Hkv, S, D, 2048, seed=41)
    q = wl.to_bf16_values(np.random.default_rng(42).standard_normal((B, Hkv * G, 512, D)).astype(np.float32))
    for kv_len in (512, 1000, 2048):
        say(f"prefill skip identity kv_len={kv_len}")
        a = run_prefill(q, K, V, kv_len)
        b = run_prefill(q, K, V, kv_len, no_skip=True)
        assert torch.equal(a, b)
        assert torch.equal(a, run_prefill(q, K, V, kv_len))     # deterministic


def test_prefill_non_causal_mask_and_garbage():
    B, Hkv, G, S, D, Lq = 1, 2, 4, 512, 128, 40
    K, V = fill_caches(kvq.INT8_TH, B, Hkv, S, D, 512, seed=51)
    q = wl.to_bf16_values(np.random.default_rng(52).standard_normal((B, Hkv * G, Lq, D)).astype(np.float32))
    kv_len = 400
    say("prefill mask")
    rng = np.random.default_rng(53)
    mask = np.where(rng.random((Lq, S)) < 0.4, -np.inf, 0.0).astype(np.float32)
    mask[:, 7] = 0.0
    ref = oracle.sdpa(q, K[1], V[1], kv_len, mask=mask, causal=False)
    got = run_prefill(q, K, V, kv_len, causal=False, mask=mask, out_dtype=torch.float32)
    check_attention(got, ref, "mask")
    # a zero mask agrees with no mask (the two bound the V scales over
    # different key sets, so they round differently); garbage past kv_len
    # has no effect (bit-identical)
    base = run_prefill(q, K, V, kv_len, causal=True)
    ref_c = oracle.sdpa(q, K[1], V[1], kv_len, causal=True)
    check_attention(base, ref_c, "no mask")
    check_attention(run_prefill(q, K, V, kv_len, causal=True, mask=np.zeros((Lq, S), np.float32)), ref_c, "zero mask")
    for dc, _ in (K, V):
        dc.codes[:, :, kv_len:] = 0xFF
        dc.scales[:, :, kv_len:] = float("nan")
        dc.zps[:, :, kv_len:] = -100
    assert torch.equal(base, run_prefill(q, K, V, kv_len, causal=True))


def test_prefill_lq1_matches_decode():
    """At Lq = 1 the causal bound is kv_len: prefill and decode agree with the
    oracle (and each other within the gate)."""
    B, Hkv, G, S, D = 2, 2, 4, 800, 128
    K, V = fill_caches(kvq.INT8_TH, B, Hkv, S, D, 800, seed=61)
    q = wl.to_bf16_values(np.random.default_rng(62).standard_normal((B, Hkv * G, 1, D)).astype(np.float32))
    say("prefill Lq=1")
    ref = oracle.sdpa(q, K[1], V[1], 777)
    check_attention(run_prefill(q, K, V, 777, out_dtype=torch.float32), ref, "prefill Lq1")
    assert torch.equal(run_prefill(q, K, V, 777, causal=True), run_prefill(q, K, V, 777, causal=False))


@pytest.mark.parametrize("qmode", [kvq.INT8_TH, kvq.UINT4_TH, kvq.MXFP4_B32])
def test_prefill_query_wide_range_in_vector(qmode):
    """q rows whose elements span 23 binades inside one vector."""
    B, Hkv, G, S, D, Lq = 1, 2, 2, 512, 128, 48
    K, V = fill_caches(qmode, B, Hkv, S, D, 400, seed=91)
    q = wide_range_q(np.random.default_rng(92), (B, Hkv * G, Lq, D))
    say(f"prefill wide-range q qmode {qmode}")
    ref = oracle.sdpa(q, K[1], V[1], 400, causal=True)
    check_attention(run_prefill(q, K, V, 400, out_dtype=torch.float32), ref, "wide q prefill")


ALL_MODES = [kvq.INT8_TH, kvq.UINT4_TH, kvq.FP8E4M3_B32, kvq.MXFP4_B32, kvq.MXFP8_B32, kvq.FP8E5M2_B32, kvq.INT8_B32,
             kvq.MXFP4E1M2_B32]


def scaled_v_caches(qmode, B, Hkv, S, D, n, vgain, seed):
    """K at unit scale, V at vgain times unit scale, written by both sides."""
    rng = np.random.default_rng(seed)
    pairs = []
    for which in range(2):
        x = rng.standard_normal((B, Hkv, n, D)).astype(np.float32)
        x[..., rng.choice(D, 4, replace=False)] *= 10
        if which == 1:
            x *= vgain
        x = wl.to_bf16_values(x)
        dc, hc = new_pair(qmode, B, Hkv, S, D)
        slots = np.broadcast_to(np.arange(n, dtype=np.int32), (B, n)).copy()
        kvq.quant_scatter(dev_input(x, True), torch.from_numpy(slots).to(DEV), dc)
        oracle.quant_scatter(hc, x, slots, parallel=True)
        pairs.append((dc, hc))
    torch.cuda.synchronize()
    for dc, hc in pairs:
        assert_cache_equal(dc, hc, "history")
    return pairs[0], pairs[1]


@pytest.mark.parametrize("vgain", [1e-3, 1e3])
@pytest.mark.parametrize("qmode", ALL_MODES)
def test_prefill_v_magnitude(qmode, vgain):
    """V far from unit scale: P * scale_v neither overflows fp16 (amax in the
    thousands gives scales in the hundreds) nor falls into its subnormals
    (amax near 1e-3).  The output is linear in V, so the gate is the unit
    gate times vgain.  The one-workgroup-per-tile kernel, the key-range split
    (the reference m goes into the partials) and a masked call."""
    B, Hkv, G, S, D, Lq, n = 1, 2, 4, 1024, 128, 128, 1000
    assert kvq.sdpa_prefill_split_workspace_bytes(B, Hkv * G, Hkv, Lq, S, D) > 0
    say(f"prefill V x{vgain} qmode {qmode}")
    K, V = scaled_v_caches(qmode, B, Hkv, S, D, n, vgain, seed=100 + qmode)
    q = wl.to_bf16_values(np.random.default_rng(101).standard_normal((B, Hkv * G, Lq, D)).astype(np.float32))
    ref = oracle.sdpa(q, K[1], V[1], n, causal=True)
    got = run_prefill(q, K, V, n, out_dtype=torch.float32)
    check_attention(got / vgain, ref / vgain, f"V x{vgain} qmode {qmode}")
    kl = torch.tensor([n], dtype=torch.int32, device=DEV)
    got = kvq.sdpa_prefill_split(dev_input(q, True), K[0], V[0], kv_len=kl, causal=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_attention(got / vgain, ref / vgain, f"split V x{vgain} qmode {qmode}")
    # with an additive mask (the scale bound then runs over the keys the mask
    # leaves visible to each row)
    mask = np.where(np.random.default_rng(102).random((Lq, S)) < 0.3, -np.inf, 0.0).astype(np.float32)
    ref = oracle.sdpa(q, K[1], V[1], n, mask=mask, causal=False)
    got = run_prefill(q, K, V, n, causal=False, mask=mask, out_dtype=torch.float32)
    check_attention(got / vgain, ref / vgain, f"masked V x{vgain} qmode {qmode}")
