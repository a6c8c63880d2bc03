"""Per-batch filled lengths and multi-token ring / sink chunks, on the GPU
against the oracle.

* kvq_sdpa_decode_varlen / kvq_sdpa_prefill_varlen: batch row b attends slots
  [0, kv_lens[b]) (pytorch/executorch PR 20351, the kv_len bound, one value
  per sequence).  Each row is compared with the oracle run on that row alone.
* Chunks of T > 1 tokens written into attention-sink and ring caches
  (pytorch/executorch PR 24473, Summary: slots from the sink / ring layout,
  an additive 0 / -inf mask from cache_positions), including chunks whose
  writes wrap the ring and chunks longer than the window, where later tokens
  of the chunk overwrite earlier ones: the step runs as positions ->
  quant-scatter -> mask (Lq = T) -> masked prefill, and every intermediate
  (slots, cache positions, cache bytes, mask) and the attention output are
  checked against the oracle running the same steps.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_kv_cache_head_amd as kvq
import quantized_kv_cache_head_amd.workloads as wl
from _gpu import DEV, assert_cache_equal, check_attention, dev_input, new_pair, say
from test_gpu_decode import fill_caches

pytestmark = pytest.mark.gpu


def _row_cache(hc, b):
    """The oracle cache of batch row b alone."""
    r = oracle.HostCache(hc.qmode, 1, hc.H, hc.S, hc.D, fill=False)
    r.codes[...] = hc.codes[b:b + 1]
    r.scales[...] = hc.scales[b:b + 1]
    if hc.zps is not None:
        r.zps[...] = hc.zps[b:b + 1]
    return r


@pytest.mark.parametrize("qmode", [kvq.INT8_TH, kvq.UINT4_TH, kvq.FP8E4M3_B32, kvq.MXFP4_B32])
def test_decode_varlen(qmode):
    B, Hkv, G, S, D = 4, 2, 4, 700, 128
    kv_lens = np.array([1, 100, 611, 700], np.int32)
    say(f"decode varlen qmode={qmode}")
    K, V = fill_caches(qmode, B, Hkv, S, D, S, seed=400 + qmode)
    q = wl.to_bf16_values(np.random.default_rng(401).standard_normal((B, Hkv * G, 1, D)).astype(np.float32))
    kl = torch.from_numpy(kv_lens).to(DEV)
    for od in (torch.float32, torch.bfloat16):
        out = kvq.sdpa_decode_varlen(dev_input(q, True), K[0], V[0], kl, out_dtype=od)
        torch.cuda.synchronize()
        for b in range(B):
            ref = oracle.sdpa(q[b:b + 1], _row_cache(K[1], b), _row_cache(V[1], b), int(kv_lens[b]))
            check_attention(out[b:b + 1], ref, f"b {b} kv_len {kv_lens[b]} {od}")
    # equal lengths: bit-identical to the one-kv_len call
    same = torch.full((B,), 611, dtype=torch.int32, device=DEV)
    a = kvq.sdpa_decode_varlen(dev_input(q, True), K[0], V[0], same)
    c = kvq.sdpa_decode(dev_input(q, True), K[0], V[0], kv_len=same[:1])
    torch.cuda.synchronize()
    assert torch.equal(a, c)


def test_decode_varlen_out_of_range_row_is_clamped_and_flagged():
    B, Hkv, G, S, D = 2, 1, 2, 256, 64
    K, V = fill_caches(kvq.INT8_TH, B, Hkv, S, D, S, seed=410)
    q = wl.to_bf16_values(np.random.default_rng(411).standard_normal((B, Hkv * G, 1, D)).astype(np.float32))
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    kl = torch.tensor([100, S + 9], dtype=torch.int32, device=DEV)
    say("decode varlen clamp")
    out = kvq.sdpa_decode_varlen(dev_input(q, True), K[0], V[0], kl, err_flags=err, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert int(err.item()) == kvq.FLAG_KVLEN
    for b, n in ((0, 100), (1, S)):
        check_attention(out[b:b + 1], oracle.sdpa(q[b:b + 1], _row_cache(K[1], b), _row_cache(V[1], b), n), f"b {b}")


@pytest.mark.parametrize("qmode", [kvq.UINT4_TH, kvq.INT8_B32])
def test_prefill_varlen(qmode):
    B, Hkv, G, S, D, Lq = 3, 2, 2, 600, 128, 64
    kv_lens = np.array([64, 300, 530], np.int32)
    say(f"prefill varlen qmode={qmode}")
    K, V = fill_caches(qmode, B, Hkv, S, D, S, seed=420 + qmode)
    q = wl.to_bf16_values(np.random.default_rng(421).standard_normal((B, Hkv * G, Lq, D)).astype(np.float32))
    out = kvq.sdpa_prefill_varlen(dev_input(q, True), K[0], V[0], torch.from_numpy(kv_lens).to(DEV),
                                  out_dtype=torch.float32)
    torch.cuda.synchronize()
    for b in range(B):
        ref = oracle.sdpa(q[b:b + 1], _row_cache(K[1], b), _row_cache(V[1], b), int(kv_lens[b]), causal=True)
        check_attention(out[b:b + 1], ref, f"b {b} kv_len {kv_lens[b]}")


@pytest.mark.parametrize("qmode", [kvq.INT8_TH, kvq.MXFP8_B32])
@pytest.mark.parametrize("sink,window,chunks", [
    (4, 60, [(0, 40), (40, 40), (80, 64), (144, 1), (145, 17)]),   # wraps; 64 > window overwrites in-chunk
    (0, 48, [(0, 30), (30, 30), (60, 48), (108, 5)]),              # ring
])
def test_ring_sink_chunks(qmode, sink, window, chunks):
    B, Hkv, G, D = 2, 2, 2, 64
    S = sink + window
    rng = np.random.default_rng(430 + sink + qmode)
    dK, hK = new_pair(qmode, B, Hkv, S, D)
    dV, hV = new_pair(qmode, B, Hkv, S, D)
    cp_dev = torch.full((S,), -1, dtype=torch.int32, device=DEV)
    cp_ref = np.full(S, -1, np.int32)
    for p0, T in chunks:
        say(f"chunk qmode={qmode} sink={sink} window={window} p0={p0} T={T}")
        start = torch.tensor([p0], dtype=torch.int32, device=DEV)
        sm = torch.empty(T, dtype=torch.int32, device=DEV)
        if sink:
            kvq.positions_with_sink(start, T, sink, window, sm, cp_dev)
        else:
            kvq.positions_ring(start, T, window, sm, cp_dev)
        sm_ref = oracle.positions_sink(p0, T, sink, window, cp_ref)
        xk = wl.to_bf16_values(rng.standard_normal((B, Hkv, T, D)).astype(np.float32))
        xv = wl.to_bf16_values(rng.standard_normal((B, Hkv, T, D)).astype(np.float32))
        kvq.quant_scatter_kv(dev_input(xk, True), dev_input(xv, True), sm, dK, dV)
        oracle.quant_scatter(hK, xk, sm_ref)
        oracle.quant_scatter(hV, xv, sm_ref)
        mask = torch.empty((T, S), dtype=torch.float32, device=DEV)
        kvq.build_mask(cp_dev, start, T, sink, window, mask)
        mask_ref = oracle.build_mask(cp_ref, p0, T, sink, window)
        kv_len = min(p0 + T, S)
        q = wl.to_bf16_values(rng.standard_normal((B, Hkv * G, T, D)).astype(np.float32))
        out = kvq.sdpa_prefill(dev_input(q, True), dK, dV, kv_len=torch.tensor([kv_len], dtype=torch.int32,
                               device=DEV), mask=mask, causal=False, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert np.array_equal(sm.cpu().numpy(), sm_ref)
        assert np.array_equal(cp_dev.cpu().numpy(), cp_ref)
        assert_cache_equal(dK, hK, "K")
        assert_cache_equal(dV, hV, "V")
        assert np.array_equal(mask.cpu().numpy(), mask_ref)
        ref = oracle.sdpa(q, hK, hV, kv_len, mask=mask_ref, causal=False)
        check_attention(out, ref, f"chunk p0 {p0} T {T}")


@pytest.mark.parametrize("qmode", [kvq.INT8_TH, kvq.MXFP4_B32])
def test_prefill_split_varlen(qmode):
    """Short chunks of a batch with one filled length per row, through the
    key-split prefill: each row against the oracle on that row alone."""
    B, Hkv, G, S, D, Lq = 3, 2, 2, 4096, 128, 24
    kv_lens = np.array([24, 1500, 4000], np.int32)
    assert kvq.sdpa_prefill_split_workspace_bytes(B, Hkv * G, Hkv, Lq, S, D) > 0
    say(f"prefill split varlen qmode={qmode}")
    K, V = fill_caches(qmode, B, Hkv, S, D, S, seed=440 + qmode)
    q = wl.to_bf16_values(np.random.default_rng(441).standard_normal((B, Hkv * G, Lq, D)).astype(np.float32))
    out = kvq.sdpa_prefill_split_varlen(dev_input(q, True), K[0], V[0], torch.from_numpy(kv_lens).to(DEV),
                                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    for b in range(B):
        ref = oracle.sdpa(q[b:b + 1], _row_cache(K[1], b), _row_cache(V[1], b), int(kv_lens[b]), causal=True)
        check_attention(out[b:b + 1], ref, f"b {b} kv_len {kv_lens[b]}")
