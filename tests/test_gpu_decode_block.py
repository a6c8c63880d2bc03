"""GPU parity of kvq_sdpa_decode over block-quantized caches (FP8-E4M3 with an
fp32 scale, MX-FP4 with an E8M0 scale, per 32 elements of a row) against the
oracle's fp64 attention on the same quantized cache: the read side of the
per-block write.  Same gate as the affine caches (2e-3, plus half a bf16 ulp
for bf16 output), same identities (data past kv_len cannot matter)."""
import numpy as np
import pytest
import torch

import oracle
import quantized_kv_cache_head_amd as kvq
import quantized_kv_cache_head_amd.workloads as wl
from _gpu import DEV, check_attention, say
from test_gpu_decode import fill_caches, run_decode

pytestmark = pytest.mark.gpu

BLOCK_MODES = [kvq.FP8E4M3_B32, kvq.MXFP4_B32, kvq.MXFP8_B32, kvq.FP8E5M2_B32, kvq.INT8_B32, kvq.MXFP4E1M2_B32]


@pytest.mark.parametrize("qmode", BLOCK_MODES)
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_block_decode_parity_shapes(qmode, D, G):
    B, Hkv, S = 2, 2, 700
    Hq = Hkv * G
    kv_len = 611                                  # several splits, ragged last step
    say(f"block decode qmode={qmode} D={D} G={G}")
    K, V = fill_caches(qmode, B, Hkv, S, D, 650, seed=D * 10 + G + 7)
    q = wl.to_bf16_values(np.random.default_rng(G + 40).standard_normal((B, Hq, 1, D)).astype(np.float32))
    ref = oracle.sdpa(q, K[1], V[1], kv_len)
    for od in (torch.bfloat16, torch.float32):
        out = run_decode(q, K, V, kv_len, out_dtype=od)
        check_attention(out, ref, f"qmode {qmode} D {D} G {G} out {od}")


@pytest.mark.parametrize("qmode", BLOCK_MODES)
def test_block_decode_fp32_query(qmode):
    B, Hkv, G, S, D = 1, 2, 4, 256, 128
    say(f"block decode fp32 q qmode={qmode}")
    K, V = fill_caches(qmode, B, Hkv, S, D, 200, seed=13, bf16=False)
    q = np.random.default_rng(14).standard_normal((B, Hkv * G, 1, D)).astype(np.float32)
    ref = oracle.sdpa(q, K[1], V[1], 200, sm_scale=0.2)
    check_attention(run_decode(q, K, V, 200, q_bf16=False, out_dtype=torch.float32, sm=0.2), ref, "fp32 q")


@pytest.mark.parametrize("qmode", BLOCK_MODES)
@pytest.mark.parametrize("kv_len", [1, 31, 33, 129, 2048])
def test_block_decode_kv_len_edges(qmode, kv_len):
    B, Hkv, G, S, D = 1, 2, 4, 2048, 128
    say(f"block decode qmode={qmode} kv_len={kv_len}")
    K, V = fill_caches(qmode, B, Hkv, S, D, kv_len, seed=kv_len + 3)
    q = wl.to_bf16_values(np.random.default_rng(kv_len).standard_normal((B, Hkv * G, 1, D)).astype(np.float32))
    ref = oracle.sdpa(q, K[1], V[1], kv_len)
    check_attention(run_decode(q, K, V, kv_len, out_dtype=torch.float32), ref, f"kv_len {kv_len}")


@pytest.mark.parametrize("qmode", BLOCK_MODES)
def test_block_decode_mask_and_past_kv_len(qmode):
    B, Hkv, G, S, D = 2, 2, 2, 512, 64
    K, V = fill_caches(qmode, B, Hkv, S, D, 512, seed=21)
    q = wl.to_bf16_values(np.random.default_rng(22).standard_normal((B, Hkv * G, 1, D)).astype(np.float32))
    kv_len = 450
    say(f"block decode identities qmode={qmode}")
    base = run_decode(q, K, V, kv_len)
    assert torch.equal(base, run_decode(q, K, V, kv_len, mask=np.zeros((1, S), np.float32)))
    # garbage past kv_len: random codes (NaN codes included), NaN / 0xFF scales
    for dc, _ in (K, V):
        dc.codes[:, :, kv_len:] = torch.randint(0, 256, dc.codes[:, :, kv_len:].shape, dtype=torch.uint8, device=DEV)
        if dc.scales.dtype == torch.uint8:
            dc.scales[:, :, kv_len:] = 0xFF
        else:
            dc.scales[:, :, kv_len:] = float("nan")
    assert torch.equal(base, run_decode(q, K, V, kv_len))
    # an additive 0 / -inf mask per batch row vs the oracle
    rng = np.random.default_rng(23)
    mask = np.where(rng.random((B, S)) < 0.3, -np.inf, 0.0).astype(np.float32)
    mask[:, 0] = 0.0
    ref = oracle.sdpa(q, K[1], V[1], kv_len, mask=mask[:, None, :])
    check_attention(run_decode(q, K, V, kv_len, out_dtype=torch.float32, mask=mask), ref, "mask")


@pytest.mark.parametrize("qmode", BLOCK_MODES)
def test_block_decode_llama_shape(qmode):
    """The Llama-3-8B-shaped decode layer (B 8, 32/8 heads, D 128, 8192 slots,
    kv_len 4096) over a block cache, in the launch configuration the
    benchmark times, against the oracle on every output."""
    w = wl.LLAMA8B
    say(f"block decode llama shape qmode={qmode}")
    K, V = fill_caches(qmode, w.B, w.Hkv, w.S, w.D, w.kv_len, seed=31)
    q = wl.to_bf16_values(np.random.default_rng(32).standard_normal((w.B, w.Hq, 1, w.D)).astype(np.float32))
    ref = oracle.sdpa(q, K[1], V[1], w.kv_len)
    check_attention(run_decode(q, K, V, w.kv_len), ref, "llama shape")


@pytest.mark.parametrize("qmode", BLOCK_MODES)
def test_block_decode_every_code(qmode):
    """With kv_len = 1 the softmax weight is exactly 1, so the fp32 output is
    the dequantized V row itself: every code of the format at scale 1 must
    come out exactly as the oracle's decoders give it.  Codes no encoder
    emits and that decode to inf / NaN (E4M3 0x7F / 0xFF, E5M2 exponent 31)
    are replaced by 0x00."""
    B, Hkv, G, S, D = 2, 1, 1, 4, 128
    say(f"block decode every code qmode={qmode}")
    K = kvq.Cache.empty(qmode, B, Hkv, S, D)
    V = kvq.Cache.empty(qmode, B, Hkv, S, D)
    if qmode in (kvq.MXFP4_B32, kvq.MXFP4E1M2_B32):
        nib = (np.arange(B * D) % 16).astype(np.uint8)
        nib = np.random.default_rng(5).permutation(nib).reshape(B, D)
        codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
        dec = oracle.e2m1_decode if qmode == kvq.MXFP4_B32 else oracle.e1m2_decode
        ref = np.array([[dec(int(c)) for c in row] for row in nib])
    else:
        codes = np.arange(256, dtype=np.uint8).reshape(B, D)
        if qmode in (kvq.FP8E4M3_B32, kvq.MXFP8_B32):
            codes[(codes & 0x7F) == 0x7F] = 0
            dec = oracle.e4m3fn_decode
        elif qmode == kvq.FP8E5M2_B32:
            codes[(codes & 0x7C) == 0x7C] = 0
            dec = oracle.e5m2_decode
        else:
            dec = lambda c: float(np.int8(np.uint8(c)))
        ref = np.array([[dec(int(c)) for c in row] for row in codes])
    for c in (K, V):
        if c.scales.dtype == torch.uint8:
            c.scales.fill_(127)                       # E8M0 2^0
        else:
            c.scales.fill_(1.0)
        c.codes.zero_()
        c.codes[:, 0, 0, :] = torch.from_numpy(codes).to(DEV)
    q = torch.zeros((B, Hkv * G, 1, D), dtype=torch.bfloat16, device=DEV)
    out = kvq.sdpa_decode(q, K, V, kv_len=torch.tensor([1], dtype=torch.int32, device=DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = out[:, 0, 0, :].cpu().numpy()
    # value equality (a -0 code sums to +0 in the accumulator)
    assert np.array_equal(got, ref.astype(np.float32)), np.argwhere(got != ref.astype(np.float32))[:8]
