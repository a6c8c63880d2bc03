"""Pins for the oracle's attention on a quantized cache.

Attention is softmax(sm_scale * q k^T + mask) v with GQA head expansion
(abaddon attention_cache, KvCache::forward_attention and repeat_kv), the KV
loop bounded by kv_len and, for causal prefill, query row r of Lq seeing keys
j <= kv_len - Lq + r (pytorch/executorch PR 20351, kv_len and per-tile causal
bound notes); ring/sink caches use the additive mask, full-context caches plain
causal attention (PR 24473, Summary).

Checked against torch's scaled_dot_product_attention in float64 (a library
routine) on the cache dequantized by plain NumPy, against closed forms
(identical keys give the mean of the visible values), and against the
invariants the pages state (data past kv_len cannot matter; Lq = 1 is the same
with and without the causal bound; GQA equals MHA on the repeated cache).
"""
import numpy as np
import pytest
import torch


def _make(orc, mode, B, Hkv, S, D, n_fill, seed):
    rng = np.random.default_rng(seed)
    x = [rng.standard_normal((B, Hkv, n_fill, D)).astype(np.float32) for _ in range(2)]
    x[0][..., :2] *= 8
    caches = []
    for xi in x:
        c = orc.HostCache(mode, B, Hkv, S, D)
        orc.quant_scatter(c, xi, np.arange(n_fill, dtype=np.int32))
        caches.append(c)
    return caches


def _dequant_numpy(orc, c, upto):
    """Plain NumPy dequantization of slots [0, upto): [B,H,upto,D] fp64."""
    codes = c.codes[:, :, :upto]
    if c.qmode == orc.INT8_TH:
        q = codes.view(np.int8).astype(np.float64)
    else:
        q = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(codes.shape[:-1] + (-1,)).astype(np.float64)
    return (q - c.zps[:, :, :upto, None]) * c.scales[:, :, :upto, :1].astype(np.float64)


def _torch_ref(q, k, v, kv_len, causal, mask, sm_scale):
    B, Hq, Lq, D = q.shape
    G = Hq // k.shape[1]
    kt = torch.from_numpy(k).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=1)
    am = torch.zeros((Lq, kv_len), dtype=torch.float64)
    if causal:
        j = torch.arange(kv_len)[None, :]
        r = torch.arange(Lq)[:, None]
        am = am.masked_fill(j > kv_len - Lq + r, float("-inf"))
    if mask is not None:
        am = am + torch.from_numpy(mask[..., :kv_len].astype(np.float64))
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), kt, vt, attn_mask=am, scale=sm_scale).numpy()


@pytest.mark.parametrize("mode_name", ["int8", "uint4"])
@pytest.mark.parametrize("Lq,kv_len,causal", [(1, 37, False), (1, 64, True), (16, 50, True), (16, 64, False)])
def test_sdpa_vs_torch(orc, mode_name, Lq, kv_len, causal):
    mode = orc.INT8_TH if mode_name == "int8" else orc.UINT4_TH
    B, Hq, Hkv, S, D = 2, 4, 2, 64, 64
    kc, vc = _make(orc, mode, B, Hkv, S, D, S, 1)
    q = np.random.default_rng(2).standard_normal((B, Hq, Lq, D))
    sm = 0.125
    got = orc.sdpa(q, kc, vc, kv_len, causal=causal, sm_scale=sm)
    want = _torch_ref(q, _dequant_numpy(orc, kc, kv_len), _dequant_numpy(orc, vc, kv_len),
                      kv_len, causal, None, sm)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_sdpa_with_mask_vs_torch(orc):
    B, Hq, Hkv, S, D, Lq = 1, 4, 2, 48, 64, 3
    kc, vc = _make(orc, orc.INT8_TH, B, Hkv, S, D, S, 3)
    cp = np.full(S, -1, np.int32)
    sm_ = orc.positions_sink(0, 60, 4, S - 4, cp)
    mask = orc.build_mask(cp, 57, Lq, 4, S - 4)
    q = np.random.default_rng(4).standard_normal((B, Hq, Lq, D))
    got = orc.sdpa(q, kc, vc, S, mask=mask, causal=False, sm_scale=0.1)
    want = _torch_ref(q, _dequant_numpy(orc, kc, S), _dequant_numpy(orc, vc, S), S, False, mask, 0.1)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    # per-batch mask layout [B, Lq, S] gives the same result
    got_b = orc.sdpa(q, kc, vc, S, mask=mask[None], causal=False, sm_scale=0.1)
    assert np.array_equal(got, got_b)


def test_identical_keys_give_mean_of_visible_values(orc):
    """Closed form: equal scores => output is the mean of the visible V rows."""
    B, Hq, Hkv, S, D, Lq, kv_len = 1, 2, 1, 32, 64, 4, 20
    rng = np.random.default_rng(8)
    kx = np.tile(rng.standard_normal((1, 1, 1, D)).astype(np.float32), (1, 1, S, 1))
    vx = rng.standard_normal((1, 1, S, D)).astype(np.float32)
    kc = orc.HostCache(orc.INT8_TH, B, Hkv, S, D)
    vc = orc.HostCache(orc.INT8_TH, B, Hkv, S, D)
    orc.quant_scatter(kc, kx, np.arange(S, dtype=np.int32))
    orc.quant_scatter(vc, vx, np.arange(S, dtype=np.int32))
    q = rng.standard_normal((B, Hq, Lq, D))
    out = orc.sdpa(q, kc, vc, kv_len, causal=True)
    vd = _dequant_numpy(orc, vc, S)[0, 0]
    for r in range(Lq):
        n_vis = kv_len - Lq + r + 1
        np.testing.assert_allclose(out[0, :, r], np.broadcast_to(vd[:n_vis].mean(0), (Hq, D)),
                                   rtol=1e-12, atol=1e-13)


def test_kv_len_bounds_the_loop(orc):
    """Slots at or past kv_len cannot change the output (bit-identical)."""
    B, Hq, Hkv, S, D = 2, 4, 2, 64, 64
    kc, vc = _make(orc, orc.INT8_TH, B, Hkv, S, D, 40, 5)     # slots 40.. are sentinel fill
    q = np.random.default_rng(6).standard_normal((B, Hq, 1, D))
    a = orc.sdpa(q, kc, vc, 40)
    rng = np.random.default_rng(7)
    kc.codes[:, :, 40:] = rng.integers(0, 256, kc.codes[:, :, 40:].shape)
    vc.scales[:, :, 40:] = 1e30
    kc.zps[:, :, 40:] = 3
    b = orc.sdpa(q, kc, vc, 40)
    assert np.array_equal(a, b) and np.all(np.isfinite(a))


def test_causal_bound_is_identity_at_lq1_and_gqa_is_repeat_kv(orc):
    B, Hq, Hkv, S, D = 1, 8, 2, 64, 64
    kc, vc = _make(orc, orc.UINT4_TH, B, Hkv, S, D, S, 9)
    q = np.random.default_rng(10).standard_normal((B, Hq, 1, D))
    assert np.array_equal(orc.sdpa(q, kc, vc, 50, causal=True), orc.sdpa(q, kc, vc, 50, causal=False))
    # MHA over the repeated cache
    G = Hq // Hkv
    kr = orc.HostCache(orc.UINT4_TH, B, Hq, S, D, fill=False)
    vr = orc.HostCache(orc.UINT4_TH, B, Hq, S, D, fill=False)
    for c, r in ((kc, kr), (vc, vr)):
        r.codes[...] = np.repeat(c.codes, G, axis=1)
        r.scales[...] = np.repeat(c.scales, G, axis=1)
        r.zps[...] = np.repeat(c.zps, G, axis=1)
    assert np.array_equal(orc.sdpa(q, kc, vc, 50), orc.sdpa(q, kr, vr, 50))


def test_fully_masked_row_is_zero_and_rows_api(orc):
    B, Hq, Hkv, S, D, Lq = 1, 2, 1, 16, 64, 2
    kc, vc = _make(orc, orc.INT8_TH, B, Hkv, S, D, S, 11)
    q = np.random.default_rng(12).standard_normal((B, Hq, Lq, D))
    mask = np.zeros((Lq, S), np.float32)
    mask[0, :] = -np.inf
    out = orc.sdpa(q, kc, vc, S, mask=mask)
    assert np.all(out[:, :, 0] == 0) and np.any(out[:, :, 1] != 0)
    rows = np.array([[0, 1, 1], [0, 0, 0]], np.int32)
    sel = orc.sdpa(q, kc, vc, S, mask=mask, rows=rows)
    assert np.array_equal(sel[0], out[0, 1, 1]) and np.array_equal(sel[1], out[0, 0, 0])
    with pytest.raises(ValueError):
        orc.sdpa(q, kc, vc, S + 1)
