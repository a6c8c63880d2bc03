"""GPU parity of kvq_quant_scatter_kv_full: the K and V update of a
full-context cache with its slots derived on the device (token t at slot
*start_pos + t; pytorch/executorch PR 20351, commit notes: the new token's K
and V go to the cache at the device-side input position).  It must write the
bytes and raise the flags of kvq_positions_full followed by
kvq_quant_scatter_kv, and the oracle's positions_full + quant_scatter, for
every mode, for chunks that run past the cache and for a negative start."""
import numpy as np
import pytest
import torch

import oracle
import quantized_kv_cache_head_amd as kvq
import quantized_kv_cache_head_amd.workloads as wl
from _gpu import DEV, assert_cache_equal, dev_input, new_pair, say

pytestmark = pytest.mark.gpu

MODES = [kvq.INT8_TH, kvq.UINT4_TH, kvq.FP8E4M3_B32, kvq.MXFP4_B32, kvq.MXFP8_B32, kvq.FP8E5M2_B32, kvq.INT8_B32,
         kvq.MXFP4E1M2_B32]


def bytes_equal(a: "kvq.Cache", b: "kvq.Cache", what):
    assert torch.equal(a.codes, b.codes), f"{what}: codes differ"
    assert torch.equal(a.scales.view(torch.uint8), b.scales.view(torch.uint8)), f"{what}: scales differ"
    if a.zps is not None:
        assert torch.equal(a.zps, b.zps), f"{what}: zero points differ"


@pytest.mark.parametrize("qmode", MODES)
@pytest.mark.parametrize("start,T", [(10, 5), (0, 1), (61, 5), (64, 3), (-3, 4), (0, 64)])
def test_scatter_kv_full(qmode, start, T):
    B, H, S, D = 2, 3, 64, 128
    say(f"scatter_kv_full qmode {qmode} start {start} T {T}")
    rng = np.random.default_rng(1000 + 7 * qmode + T)
    xk = wl.to_bf16_values(rng.standard_normal((B, H, T, D)).astype(np.float32))
    xv = wl.to_bf16_values(rng.standard_normal((B, H, T, D)).astype(np.float32))
    (K1, hk), (V1, hv) = new_pair(qmode, B, H, S, D), new_pair(qmode, B, H, S, D)
    (K2, _), (V2, _) = new_pair(qmode, B, H, S, D), new_pair(qmode, B, H, S, D)
    sp = torch.tensor([start], dtype=torch.int32, device=DEV)
    f1 = torch.zeros(1, dtype=torch.int32, device=DEV)
    f2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    xkd, xvd = dev_input(xk, True), dev_input(xv, True)
    # fused
    kvq.quant_scatter_kv_full(xkd, xvd, sp, K1, V1, err_flags=f1)
    # two launches
    slot = torch.empty(T, dtype=torch.int32, device=DEV)
    kvq.positions_full(sp, T, S, slot, err_flags=f2)
    kvq.quant_scatter_kv(xkd, xvd, slot, K2, V2, err_flags=f2)
    torch.cuda.synchronize()
    bytes_equal(K1, K2, "K vs two launches")
    bytes_equal(V1, V2, "V vs two launches")
    assert int(f1.item()) == int(f2.item())
    if start < 0:
        # the rejected start (the boundary's error rule; the pages have no
        # negative positions): nothing written, the slot-range flag
        assert_cache_equal(K1, hk, "K untouched")
        assert_cache_equal(V1, hv, "V untouched")
        assert int(f1.item()) == kvq.FLAG_SLOT_RANGE
        return
    # the oracle
    sm, pflags = oracle.positions_full(start, T, S)
    sflags = oracle.quant_scatter(hk, xk, sm)
    oracle.quant_scatter(hv, xv, sm)
    assert_cache_equal(K1, hk, "K vs oracle")
    assert_cache_equal(V1, hv, "V vs oracle")
    assert int(f1.item()) == (pflags | sflags)
    if start + T > S:
        assert int(f1.item()) == kvq.FLAG_POS_CAPACITY
    else:
        assert int(f1.item()) == 0


def test_scatter_kv_full_fp32_strided():
    """fp32 inputs in a strided view ([B, T, H, D] storage read as [B, H, T, D])."""
    B, H, S, D, T, start = 2, 4, 40, 64, 6, 30
    rng = np.random.default_rng(77)
    base_k = rng.standard_normal((B, T, H, D)).astype(np.float32)
    base_v = rng.standard_normal((B, T, H, D)).astype(np.float32)
    xkd = torch.from_numpy(base_k).to(DEV).transpose(1, 2)
    xvd = torch.from_numpy(base_v).to(DEV).transpose(1, 2)
    (K, hk), (V, hv) = new_pair(kvq.INT8_TH, B, H, S, D), new_pair(kvq.INT8_TH, B, H, S, D)
    say("scatter_kv_full fp32 strided")
    kvq.quant_scatter_kv_full(xkd, xvd, torch.tensor([start], dtype=torch.int32, device=DEV), K, V)
    torch.cuda.synchronize()
    sm, _ = oracle.positions_full(start, T, S)
    oracle.quant_scatter(hk, base_k.transpose(0, 2, 1, 3), sm)
    oracle.quant_scatter(hv, base_v.transpose(0, 2, 1, 3), sm)
    assert_cache_equal(K, hk, "K")
    assert_cache_equal(V, hv, "V")
