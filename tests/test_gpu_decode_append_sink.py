"""GPU parity of kvq_sdpa_decode_append_sink (the one-launch decode step of a
sink or ring int8 cache).

Its definition is the four-call sequence kvq_positions_with_sink ->
kvq_quant_scatter_kv -> kvq_build_mask -> kvq_sdpa_decode(kv_len =
min(p + 1, n_slots), mask); every case checks, on the same inputs, that the
one launch leaves the same cache bytes and cache_positions as the four calls
and gives the same output bits and flags, and that cache bytes,
cache_positions and output agree with the oracle's positions, quant-scatter,
mask and fp64 attention.  Positions cover the sink slots, the first pass
through the window, the first wrap, a later wrap, and a negative start."""
import numpy as np
import pytest
import torch

import oracle
import quantized_kv_cache_head_amd as kvq
import quantized_kv_cache_head_amd.workloads as wl
from _gpu import DEV, assert_cache_equal, check_attention, dev_input, new_pair, say

pytestmark = pytest.mark.gpu


def clone(c: kvq.Cache) -> kvq.Cache:
    return kvq.Cache(c.qmode, c.B, c.H, c.S, c.D, c.codes.clone(), c.scales.clone(), c.zps.clone())


def bf16_rows(rng, shape, outlier=True):
    x = rng.standard_normal(shape).astype(np.float32)
    if outlier:
        x[..., 5] *= 10
    return wl.to_bf16_values(x)


def history(B, Hkv, sink, window, D, p, rng):
    """Caches and cache_positions as a stream of single-token steps leaves
    them before position p: the sink positions and the last `window` others,
    written through the positions manager (GPU and oracle, checked equal)."""
    S = sink + window
    cp_d = torch.full((S,), -1, dtype=torch.int32, device=DEV)
    cp_h = np.full(S, -1, np.int32)
    pairs = [new_pair(kvq.INT8_TH, B, Hkv, S, D) for _ in range(2)]
    runs = []
    if p > 0:
        runs.append((0, min(sink, p)))
        lo = max(sink, p - window)
        if p > lo:
            runs.append((lo, p - lo))
    for start, T in runs:
        if T <= 0:
            continue
        sm_d = torch.empty(T, dtype=torch.int32, device=DEV)
        kvq.positions_with_sink(torch.tensor([start], dtype=torch.int32, device=DEV), T, sink, window, sm_d, cp_d)
        sm_h = oracle.positions_sink(start, T, sink, window, cp_h)
        assert np.array_equal(sm_d.cpu().numpy(), sm_h)
        for dc, hc in pairs:
            x = bf16_rows(rng, (B, Hkv, T, D))
            kvq.quant_scatter(dev_input(x, True), sm_d, dc)
            oracle.quant_scatter(hc, x, sm_h)
    torch.cuda.synchronize()
    for dc, hc in pairs:
        assert_cache_equal(dc, hc, "history")
    assert np.array_equal(cp_d.cpu().numpy(), cp_h)
    return pairs, cp_d, cp_h


def one_step(q_np, xk_np, xv_np, p, sink, window, K, V, cp_d, hK, hV, cp_h, ws, out_dtype=torch.bfloat16):
    """The step at position p both ways and by the oracle; the caches (K, V,
    cp_d, hK, hV, cp_h) advance by the fused call / the oracle."""
    S = sink + window
    B, Hq = q_np.shape[:2]
    q = dev_input(q_np, True)
    xk, xv = dev_input(xk_np, True), dev_input(xv_np, True)
    sp = torch.tensor([p], dtype=torch.int32, device=DEV)
    K2, V2, cp2 = clone(K), clone(V), cp_d.clone()
    err2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    slot = torch.empty(1, dtype=torch.int32, device=DEV)
    mask = torch.empty((1, S), dtype=torch.float32, device=DEV)
    kvq.positions_with_sink(sp, 1, sink, window, slot, cp2, err_flags=err2)
    kvq.quant_scatter_kv(xk, xv, slot, K2, V2, err_flags=err2)
    kvq.build_mask(cp2, sp, 1, sink, window, mask)
    kl = torch.tensor([min(p + 1, S)], dtype=torch.int32, device=DEV)
    out2 = kvq.sdpa_decode(q, K2, V2, kv_len=kl, mask=mask, out_dtype=out_dtype, err_flags=err2)
    err1 = torch.zeros(1, dtype=torch.int32, device=DEV)
    out1 = kvq.sdpa_decode_append_sink(q, xk, xv, sp, sink, window, cp_d, K, V, out_dtype=out_dtype,
                                       workspace=ws, err_flags=err1)
    torch.cuda.synchronize()
    assert int(err1.item()) == int(err2.item()), (int(err1.item()), int(err2.item()))
    assert torch.equal(cp_d, cp2), "cache_positions differ from the four-call sequence"
    for a, b, what in ((K, K2, "K"), (V, V2, "V")):
        assert torch.equal(a.codes, b.codes), f"{what} codes differ from the four-call sequence"
        assert torch.equal(a.scales.view(torch.int32), b.scales.view(torch.int32)), f"{what} scales differ"
        assert torch.equal(a.zps, b.zps), f"{what} zero points differ"
    iv = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
    assert torch.equal(out1.view(iv), out2.view(iv)), "output differs from the four-call sequence"
    # the oracle
    if p >= 0:
        sm = oracle.positions_sink(p, 1, sink, window, cp_h)
        oracle.quant_scatter(hK, xk_np, sm)
        oracle.quant_scatter(hV, xv_np, sm)
    assert np.array_equal(cp_d.cpu().numpy(), cp_h), "cache_positions differ from the oracle"
    assert_cache_equal(K, hK, f"K after the step at {p}")
    assert_cache_equal(V, hV, f"V after the step at {p}")
    m = oracle.build_mask(cp_h, p, 1, sink, window)
    ref = oracle.sdpa(q_np, hK, hV, min(max(p + 1, 1), S), mask=m)
    check_attention(out1, ref, f"append sink step at {p}")
    return int(err1.item())


def case(sink, window, B, Hkv, G, D, p, seed, out_dtype=torch.bfloat16):
    say(f"decode append sink {sink} window {window} B{B} Hkv{Hkv} G{G} D{D} position {p}")
    rng = np.random.default_rng(seed)
    pairs, cp_d, cp_h = history(B, Hkv, sink, window, D, p, rng)
    (K, hK), (V, hV) = pairs
    ws = kvq.decode_workspace(B, Hkv * G, Hkv, sink + window, D, DEV)
    q_np = bf16_rows(rng, (B, Hkv * G, 1, D), outlier=False)
    return one_step(q_np, bf16_rows(rng, (B, Hkv, 1, D)), bf16_rows(rng, (B, Hkv, 1, D)), p, sink, window,
                    K, V, cp_d, hK, hV, cp_h, ws, out_dtype)


@pytest.mark.parametrize("p", [0, 3, 4, 300, 511, 512, 515, 1500])
def test_append_sink_positions(p):
    assert case(4, 508, 2, 2, 4, 128, p, seed=p) == 0


@pytest.mark.parametrize("p", [0, 255, 256, 1000])
def test_append_ring_positions(p):
    assert case(0, 256, 2, 2, 4, 128, p, seed=100 + p, out_dtype=torch.float32) == 0


@pytest.mark.parametrize("D,G", [(64, 8), (256, 4), (128, 1)])
def test_append_sink_shapes(D, G):
    assert case(4, 508, 2, 2, G, D, 777, seed=D + G) == 0


def test_append_sink_negative_start():
    assert case(4, 508, 2, 2, 4, 128, -1, seed=9) == kvq.FLAG_SLOT_RANGE | kvq.FLAG_KVLEN


def test_append_sink_c3_shape_steps_across_the_wrap():
    """The sink cache of the sink / ring workload (B 4, 32 / 8 heads, D 128,
    sink 4 + window 2044): twelve steps in a row on the same caches through
    the first wrap of the window (positions 2042 .. 2053)."""
    sink, window, B, Hkv, G, D = 4, 2044, 4, 8, 4, 128
    rng = np.random.default_rng(6000)
    pairs, cp_d, cp_h = history(B, Hkv, sink, window, D, 2042, rng)
    (K, hK), (V, hV) = pairs
    ws = kvq.decode_workspace(B, Hkv * G, Hkv, sink + window, D, DEV)
    for p in range(2042, 2054):
        say(f"sink step {p}")
        q_np = bf16_rows(rng, (B, Hkv * G, 1, D), outlier=False)
        assert one_step(q_np, bf16_rows(rng, (B, Hkv, 1, D)), bf16_rows(rng, (B, Hkv, 1, D)), p, sink, window,
                        K, V, cp_d, hK, hV, cp_h, ws) == 0
