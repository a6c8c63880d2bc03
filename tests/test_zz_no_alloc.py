"""kvq_sdpa_decode_noalloc (decode on the library's own per-GPU scratch
array, for callers that cannot allocate) against kvq_sdpa_decode with a
caller workspace: bit-identical outputs on the same inputs, since both run
the same kernels with the same split count and merge order; and within the
attention tolerance of the fp64 oracle.  Calls in a row of different shapes
(a smaller one after a larger, then the larger again) check that the shared
array carries nothing from one call into the next."""
import numpy as np
import pytest
import torch

import oracle
import quantized_kv_cache_head_amd as kvq
import quantized_kv_cache_head_amd.workloads as wl
from _gpu import DEV, assert_cache_equal, check_attention, dev_input, new_pair, say

pytestmark = pytest.mark.gpu


def caches(qmode, B, Hkv, S, D, n_fill, seed):
    rng = np.random.default_rng(seed)
    pairs = []
    for _ in range(2):
        x = rng.standard_normal((B, Hkv, n_fill, D)).astype(np.float32)
        x[..., rng.choice(D, 4, replace=False)] *= 10
        x = wl.to_bf16_values(x)
        dc, hc = new_pair(qmode, B, Hkv, S, D)
        slots = np.broadcast_to(np.arange(n_fill, dtype=np.int32), (B, n_fill)).copy()
        kvq.quant_scatter(dev_input(x, True), torch.from_numpy(slots).to(DEV), dc)
        oracle.quant_scatter(hc, x, slots, parallel=True)
        pairs.append((dc, hc))
    torch.cuda.synchronize()
    for dc, hc in pairs:
        assert_cache_equal(dc, hc, "history")
    return pairs


def one_call(qmode, q_bf16, B, Hkv, G, S, D, kv_len, seed, masked):
    say(f"noalloc decode qmode {qmode} bf16 q {q_bf16} B{B} Hkv{Hkv} G{G} S{S} D{D} kv_len {kv_len} mask {masked}")
    K, V = caches(qmode, B, Hkv, S, D, kv_len, seed)
    rng = np.random.default_rng(seed + 1)
    q_np = rng.standard_normal((B, Hkv * G, 1, D)).astype(np.float32)
    if q_bf16:
        q_np = wl.to_bf16_values(q_np)
    q = dev_input(q_np, q_bf16)
    kl = torch.tensor([kv_len], dtype=torch.int32, device=DEV)
    mask_np = None
    if masked:
        mask_np = np.where(rng.random((B, S)) < 0.2, -np.inf, 0.0).astype(np.float32)
        mask_np[:, kv_len - 1] = 0.0
    md = None if mask_np is None else torch.from_numpy(mask_np).to(DEV)
    ref = oracle.sdpa(q_np, K[1], V[1], kv_len, mask=None if mask_np is None else mask_np[:, None, :])
    for od in (torch.float32, torch.bfloat16):
        err_a = torch.zeros(1, dtype=torch.int32, device=DEV)
        err_b = torch.zeros(1, dtype=torch.int32, device=DEV)
        a = kvq.sdpa_decode(q, K[0], V[0], kv_len=kl, mask=md, out_dtype=od, err_flags=err_a)
        b = kvq.sdpa_decode_noalloc(q, K[0], V[0], kv_len=kl, mask=md, out_dtype=od, err_flags=err_b)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16) if od == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if od == torch.bfloat16 else b.view(torch.int32)), \
            f"noalloc differs from the workspace entry point ({od})"
        assert int(err_a.item()) == int(err_b.item()) == 0
        check_attention(b, ref, f"noalloc qmode {qmode} {od}")


@pytest.mark.parametrize("q_bf16", [True, False])
@pytest.mark.parametrize("qmode", [kvq.INT8_TH, kvq.UINT4_TH, kvq.FP8E4M3_B32])
def test_noalloc_matches_workspace_decode(qmode, q_bf16):
    # larger, then smaller (fewer tickets, fewer partials), then larger again
    one_call(qmode, q_bf16, B=4, Hkv=8, G=4, S=2048, D=128, kv_len=1531, seed=7, masked=False)
    one_call(qmode, q_bf16, B=2, Hkv=2, G=2, S=256, D=64, kv_len=200, seed=8, masked=True)
    one_call(qmode, q_bf16, B=4, Hkv=8, G=4, S=2048, D=128, kv_len=1531, seed=9, masked=True)


def test_noalloc_rejects_oversized_call():
    # B * Hq * (D + 2) * 4 bytes of partials for even one split exceed the
    # partial region: rejected on the host, nothing enqueued
    B, Hkv, G, S, D = 256, 8, 8, 16, 256
    k = kvq.Cache.empty(kvq.INT8_TH, B, Hkv, S, D)
    v = kvq.Cache.empty(kvq.INT8_TH, B, Hkv, S, D)
    q = torch.zeros((B, Hkv * G, 1, D), dtype=torch.bfloat16, device=DEV)
    say("noalloc decode oversized call")
    with pytest.raises(kvq.KvqError) as e:
        kvq.sdpa_decode_noalloc(q, k, v)
    assert e.value.status == 5
    torch.cuda.synchronize()
