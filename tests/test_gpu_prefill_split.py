"""GPU parity of kvq_sdpa_prefill_split -- chunked prefill with each query
tile's key range split over several workgroups and the partials merged per
query row -- against the oracle's fp64 attention on the same quantized cache
(pytorch/executorch PR 20351: chunked prefill, kv_len bound, per-tile causal
bound).  Short chunks (few query tiles), splits that end up empty under the
causal bound, masks, every cache family; large chunks, where no split is
used, must match kvq_sdpa_prefill bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import quantized_kv_cache_head_amd as kvq
import quantized_kv_cache_head_amd.workloads as wl
from _gpu import DEV, check_attention, say
from test_gpu_decode import fill_caches

pytestmark = pytest.mark.gpu

MODES = [kvq.INT8_TH, kvq.UINT4_TH, kvq.FP8E4M3_B32, kvq.MXFP4_B32]


def _q(rng, B, Hq, Lq, D):
    return wl.to_bf16_values(rng.standard_normal((B, Hq, Lq, D)).astype(np.float32))


def _run(q, K, V, kv_len, split=True, **kw):
    f = kvq.sdpa_prefill_split if split else kvq.sdpa_prefill
    out = f(torch.from_numpy(q).to(torch.bfloat16).to(DEV), K[0], V[0],
            kv_len=torch.tensor([kv_len], dtype=torch.int32, device=DEV), **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("qmode", MODES)
@pytest.mark.parametrize("Lq,kv_len", [(1, 1), (1, 3000), (16, 700), (64, 4096), (100, 2500)])
def test_split_prefill_parity(qmode, Lq, kv_len):
    B, Hkv, G, S, D = 1, 2, 2, 4096, 128
    assert kvq.sdpa_prefill_split_workspace_bytes(B, Hkv * G, Hkv, Lq, S, D) > 0   # the split path runs
    say(f"split prefill qmode={qmode} Lq={Lq} kv_len={kv_len}")
    K, V = fill_caches(qmode, B, Hkv, S, D, kv_len, seed=Lq * 7 + kv_len + qmode)
    q = _q(np.random.default_rng(Lq + kv_len), B, Hkv * G, Lq, D)
    ref = oracle.sdpa(q, K[1], V[1], kv_len, causal=True)
    for od in (torch.float32, torch.bfloat16):
        check_attention(_run(q, K, V, kv_len, out_dtype=od), ref, f"qmode {qmode} Lq {Lq} kv {kv_len} {od}")


@pytest.mark.parametrize("D,G", [(64, 1), (64, 8), (256, 2), (128, 4)])
def test_split_prefill_shapes(D, G):
    B, Hkv, S, Lq, kv_len = 2, 2, 3000, 40, 2900
    say(f"split prefill D={D} G={G}")
    K, V = fill_caches(kvq.INT8_TH, B, Hkv, S, D, kv_len, seed=D + G)
    q = _q(np.random.default_rng(D * G), B, Hkv * G, Lq, D)
    ref = oracle.sdpa(q, K[1], V[1], kv_len, causal=True)
    check_attention(_run(q, K, V, kv_len, out_dtype=torch.float32), ref, f"D {D} G {G}")


def test_split_prefill_mask_and_non_causal():
    B, Hkv, G, S, D, Lq, kv_len = 1, 2, 4, 2048, 128, 24, 2000
    say("split prefill mask")
    K, V = fill_caches(kvq.UINT4_TH, B, Hkv, S, D, kv_len, seed=5)
    q = _q(np.random.default_rng(6), B, Hkv * G, Lq, D)
    rng = np.random.default_rng(7)
    mask = np.where(rng.random((Lq, S)) < 0.5, -np.inf, 0.0).astype(np.float32)
    mask[:, 0] = 0.0
    ref = oracle.sdpa(q, K[1], V[1], kv_len, mask=mask, causal=False)
    got = _run(q, K, V, kv_len, mask=torch.from_numpy(mask).to(DEV), causal=False, out_dtype=torch.float32)
    check_attention(got, ref, "mask")
    # a row whose every key is masked gives 0 through the merge as well
    mask[3, :] = -np.inf
    got = _run(q, K, V, kv_len, mask=torch.from_numpy(mask).to(DEV), causal=False, out_dtype=torch.float32)
    assert torch.count_nonzero(got[0, :, 3]) == 0


def test_split_prefill_without_split_is_prefill():
    """Chunks whose query tiles fill the part take no workspace and give the
    bits of kvq_sdpa_prefill."""
    B, Hkv, G, S, D, Lq, kv_len = 1, 16, 2, 4096, 256, 2048, 4096
    assert kvq.sdpa_prefill_split_workspace_bytes(B, Hkv * G, Hkv, Lq, S, D) == 0
    say("split prefill = prefill for a full chunk")
    K, V = fill_caches(kvq.UINT4_TH, B, Hkv, S, D, kv_len, seed=9)
    q = _q(np.random.default_rng(10), B, Hkv * G, Lq, D)
    assert torch.equal(_run(q, K, V, kv_len), _run(q, K, V, kv_len, split=False))


def test_split_prefill_small_workspace_raises():
    B, Hkv, G, S, D, Lq = 1, 2, 2, 4096, 128, 16
    K, V = fill_caches(kvq.INT8_TH, B, Hkv, S, D, S, seed=11)
    q = torch.zeros((B, Hkv * G, Lq, D), dtype=torch.bfloat16, device=DEV)
    need = kvq.sdpa_prefill_split_workspace_bytes(B, Hkv * G, Hkv, Lq, S, D)
    ws = torch.empty(need - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(RuntimeError):
        kvq.sdpa_prefill_split(q, K[0], V[0], workspace=ws)


@pytest.mark.parametrize("qmode", [kvq.INT8_TH, kvq.MXFP8_B32])
def test_split_prefill_causal_skip_identity_and_fp32(qmode):
    """Split boundaries follow kv_len, so scanning every tile below kv_len
    (KVQ_NO_CAUSAL_SKIP) gives the same bits as stopping at the per-tile causal
    bound; fp32 queries (hi + lo limbs) through the split path against the
    oracle."""
    B, Hkv, G, S, D, Lq, kv_len = 1, 2, 4, 4096, 128, 200, 3000
    say(f"split prefill skip identity qmode={qmode}")
    K, V = fill_caches(qmode, B, Hkv, S, D, kv_len, seed=12 + qmode)
    q = _q(np.random.default_rng(13), B, Hkv * G, Lq, D)
    assert torch.equal(_run(q, K, V, kv_len), _run(q, K, V, kv_len, no_causal_skip=True))
    q32 = np.random.default_rng(14).standard_normal((B, Hkv * G, Lq, D)).astype(np.float32)
    out = kvq.sdpa_prefill_split(torch.from_numpy(q32).to(DEV), K[0], V[0],
                                 kv_len=torch.tensor([kv_len], dtype=torch.int32, device=DEV),
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_attention(out, oracle.sdpa(q32, K[1], V[1], kv_len, causal=True), "fp32 q")
