"""A slot that the additive mask hides takes no part in attention, whatever
its scale holds (pytorch/executorch PR 24473, Summary: ring and sink caches
attend through an additive 0 / -inf mask).  A ring cache that is not full yet
holds sentinel bytes in its unwritten slots (NaN fp32 scales, 0xFF E8M0
scales, 0x5A zero points, 0xA5 codes); decode and chunked prefill over the
whole cache (kv_len = n_slots) with the mask that hides those slots must give
what the oracle gives, which skips masked keys."""
import numpy as np
import pytest
import torch

import oracle
import quantized_kv_cache_head_amd as kvq
import quantized_kv_cache_head_amd.workloads as wl
from _gpu import DEV, assert_cache_equal, check_attention, dev_input, new_pair, say

pytestmark = pytest.mark.gpu

MODES = [kvq.INT8_TH, kvq.UINT4_TH, kvq.FP8E4M3_B32, kvq.MXFP4_B32, kvq.MXFP8_B32, kvq.MXFP4E1M2_B32]


def ring_caches(qmode, B, Hkv, S, D, written, seed):
    """K and V ring caches whose slots [0, written) hold positions 0..written-1
    (written by the GPU kernel and by the oracle from the same inputs); the
    other slots keep the sentinel fill."""
    rng = np.random.default_rng(seed)
    pairs = []
    for _ in range(2):
        x = wl.to_bf16_values(rng.standard_normal((B, Hkv, written, D)).astype(np.float32))
        dc, hc = new_pair(qmode, B, Hkv, S, D)
        slots = np.broadcast_to(np.arange(written, dtype=np.int32), (B, written)).copy()
        kvq.quant_scatter(dev_input(x, True), torch.from_numpy(slots).to(DEV), dc)
        oracle.quant_scatter(hc, x, slots)
        pairs.append((dc, hc))
    torch.cuda.synchronize()
    for dc, hc in pairs:
        assert_cache_equal(dc, hc, "ring history")
    return pairs


def ring_positions(S, written):
    cp = np.full(S, -1, np.int32)
    cp[:written] = np.arange(written, dtype=np.int32)
    return cp


@pytest.mark.parametrize("qmode", MODES)
def test_decode_mask_hides_unwritten_slots(qmode):
    B, Hkv, G, S, D, written = 2, 2, 4, 256, 128, 100
    say(f"decode over a part-filled ring cache, qmode {qmode}")
    K, V = ring_caches(qmode, B, Hkv, S, D, written, seed=31 + qmode)
    # the query sits at the last written position; a window of S slots
    mask = oracle.build_mask(ring_positions(S, written), written - 1, 1, 0, S)      # [1, S]
    assert np.isneginf(mask[0, written:]).all() and (mask[0, :written] == 0).all()
    q = wl.to_bf16_values(np.random.default_rng(32).standard_normal((B, Hkv * G, 1, D)).astype(np.float32))
    ref = oracle.sdpa(q, K[1], V[1], S, mask=mask)
    md = torch.from_numpy(mask).to(DEV)
    for od in (torch.float32, torch.bfloat16):
        out = kvq.sdpa_decode(dev_input(q, True), K[0], V[0], kv_len=None, mask=md, out_dtype=od)
        torch.cuda.synchronize()
        check_attention(out, ref, f"decode qmode {qmode} {od}")


@pytest.mark.parametrize("qmode", MODES)
def test_prefill_mask_hides_unwritten_slots(qmode):
    B, Hkv, G, S, D, written, Lq = 1, 2, 2, 256, 128, 90, 24
    say(f"prefill over a part-filled ring cache, qmode {qmode}")
    K, V = ring_caches(qmode, B, Hkv, S, D, written, seed=41 + qmode)
    # the chunk's rows are the last Lq written positions; the mask carries
    # both causality and the unwritten slots
    p0 = written - Lq
    mask = oracle.build_mask(ring_positions(S, written), p0, Lq, 0, S)              # [Lq, S]
    q = wl.to_bf16_values(np.random.default_rng(42).standard_normal((B, Hkv * G, Lq, D)).astype(np.float32))
    ref = oracle.sdpa(q, K[1], V[1], S, mask=mask, causal=False)
    md = torch.from_numpy(mask).to(DEV)
    for od in (torch.float32, torch.bfloat16):
        out = kvq.sdpa_prefill(dev_input(q, True), K[0], V[0], kv_len=None, mask=md, causal=False, out_dtype=od)
        torch.cuda.synchronize()
        check_attention(out, ref, f"prefill qmode {qmode} {od}")
