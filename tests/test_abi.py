"""CPU checks of the C-ABI library: it loads, exports every entry point that
include/kvq.h declares, and rejects bad arguments on the host (no GPU work is
started by any call here: each one fails validation before a launch)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def kvq():
    import quantized_kv_cache_head_amd as kvq
    if not os.path.exists(kvq.LIB_PATH):
        from quantized_kv_cache_head_amd import build
        build.build()
    kvq.lib()
    return kvq


def _declared():
    text = open(os.path.join(ROOT, "include", "kvq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree(kvq):
    assert _declared() == sorted(kvq.EXPORTS)


def test_every_declared_symbol_is_exported(kvq):
    out = subprocess.run(["nm", "-D", "--defined-only", kvq.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (kvq_\w+)", out))
    for name in _declared():
        assert name in exported, name
        assert hasattr(kvq.lib(), name)
    # nothing else leaks out of the library
    assert exported == set(_declared())


def test_status_strings(kvq):
    for st in range(7):
        assert kvq.status_string(st)
    assert kvq.status_string(0) == "ok"


def test_cache_bytes(kvq):
    assert kvq.cache_bytes(kvq.INT8_TH, 8, 8, 8192, 128) == (8 * 8 * 8192 * 128, 8 * 8 * 8192 * 4, 8 * 8 * 8192)
    assert kvq.cache_bytes(kvq.UINT4_TH, 1, 16, 131072, 256) == (16 * 131072 * 128, 16 * 131072 * 4, 16 * 131072)
    assert kvq.cache_bytes(kvq.FP8E4M3_B32, 1, 1, 65536, 128) == (65536 * 128, 65536 * 4 * 4, 0)
    assert kvq.cache_bytes(kvq.MXFP4_B32, 1, 1, 65536, 128) == (65536 * 64, 65536 * 4, 0)
    assert kvq.cache_bytes(kvq.MXFP8_B32, 1, 1, 65536, 128) == (65536 * 128, 65536 * 4, 0)
    assert kvq.cache_bytes(kvq.FP8E5M2_B32, 1, 1, 65536, 128) == (65536 * 128, 65536 * 4 * 4, 0)
    assert kvq.cache_bytes(kvq.INT8_B32, 1, 1, 65536, 128) == (65536 * 128, 65536 * 4 * 4, 0)
    assert kvq.cache_bytes(kvq.MXFP4E1M2_B32, 1, 1, 65536, 128) == (65536 * 64, 65536 * 4, 0)
    with pytest.raises(kvq.KvqError):
        kvq.cache_bytes(kvq.FP8E4M3_B32, 1, 1, 16, 48)        # D % 32 != 0
    with pytest.raises(kvq.KvqError):
        kvq.cache_bytes(kvq.UINT4_TH, 1, 1, 16, 60)           # D % 8 != 0
    with pytest.raises(kvq.KvqError):
        kvq.cache_bytes(8, 1, 1, 16, 64)                      # no such mode


def _fake_cache(kvq, qmode=0, B=1, H=2, S=64, D=64, zps=True):
    # host addresses are never dereferenced: every call below fails validation
    buf = ctypes.create_string_buffer(1 << 16)
    base = (ctypes.addressof(buf) + 255) & ~255
    c = kvq.kvq_cache(qmode, B, H, S, D, base, base, base if zps else 0)
    return c, buf


def test_noalloc_decode_validation(kvq):
    """kvq_sdpa_decode_noalloc rejects on the host, before it touches the
    device: bad shapes as kvq_sdpa_decode does, and more tickets than its
    fixed counter block holds (B * heads above 16384) as a workspace error."""
    L = kvq.lib()
    c, keep = _fake_cache(kvq)
    q = ctypes.c_void_p(c.codes)
    s = None
    assert L.kvq_sdpa_decode_noalloc(q, 1, 1, 3, ctypes.byref(c), ctypes.byref(c), None, None, 0, 0, 0.1, q, 1,
                                     None, s) == 2
    assert L.kvq_sdpa_decode_noalloc(q, 1, 1, 4, ctypes.byref(c), ctypes.byref(c), None, None, -1, 0, 0.1, q, 1,
                                     None, s) == 2
    assert L.kvq_sdpa_decode_noalloc(None, 1, 1, 4, ctypes.byref(c), ctypes.byref(c), None, None, 0, 0, 0.1, q, 1,
                                     None, s) == 1
    big, keep2 = _fake_cache(kvq, B=4096, H=8)
    assert L.kvq_sdpa_decode_noalloc(q, 1, 4096, 32, ctypes.byref(big), ctypes.byref(big), None, None, 0, 0, 0.1,
                                     q, 1, None, s) == 5


def test_host_validation_errors(kvq):
    L = kvq.lib()
    c, keep = _fake_cache(kvq)
    s = None
    # NULL cache / NULL x
    assert L.kvq_quant_scatter(None, 1, 1, 2, 4, 64, 0, 0, 64, None, 0, None, None, s) == 1
    assert L.kvq_quant_scatter(None, 1, 1, 2, 4, 64, 0, 0, 64, None, 0, ctypes.byref(c), None, s) == 1
    # shape mismatch with the cache
    assert L.kvq_quant_scatter(None, 1, 1, 3, 4, 64, 0, 0, 64, None, 0, ctypes.byref(c), None, s) == 2
    # bad dtype
    assert L.kvq_quant_scatter(None, 5, 1, 2, 4, 64, 0, 0, 64, None, 0, ctypes.byref(c), None, s) == 3
    # T == 0 is a no-op
    assert L.kvq_quant_scatter(None, 1, 1, 2, 0, 64, 0, 0, 64, None, 0, ctypes.byref(c), None, s) == 0
    # affine cache without zero points
    cz, keep2 = _fake_cache(kvq, zps=False)
    assert L.kvq_quant_scatter(None, 1, 1, 2, 4, 64, 0, 0, 64, None, 0, ctypes.byref(cz), None, s) == 1
    # quantize options: unknown bits, and the MX scale option on a non-MX cache
    cf8, keep7 = _fake_cache(kvq, qmode=kvq.FP8E4M3_B32, zps=False)
    cmx, keep8 = _fake_cache(kvq, qmode=kvq.MXFP8_B32, zps=False)
    assert L.kvq_quant_scatter_flags(None, 1, 1, 2, 4, 64, 0, 0, 64, None, 0, ctypes.byref(cf8), 1, None, s) == 4
    assert L.kvq_quant_scatter_flags(None, 1, 1, 2, 4, 64, 0, 0, 64, None, 0, ctypes.byref(cmx), 2, None, s) == 4
    assert L.kvq_quant_scatter_flags(None, 1, 1, 2, 0, 64, 0, 0, 64, None, 0, ctypes.byref(cmx), 1, None, s) == 0
    # K+V update: the two caches must agree in mode and sizes
    cv_other, keep5 = _fake_cache(kvq, S=32)
    assert L.kvq_quant_scatter_kv(None, None, 1, 1, 2, 4, 64, 0, 0, 64, None, 0, ctypes.byref(c),
                                  ctypes.byref(cv_other), None, s) == 2
    assert L.kvq_quant_scatter_kv(None, None, 1, 1, 2, 4, 64, 0, 0, 64, None, 0, ctypes.byref(c),
                                  ctypes.byref(c), None, s) == 1
    assert L.kvq_quant_scatter_kv(None, None, 1, 1, 2, 0, 64, 0, 0, 64, None, 0, ctypes.byref(c),
                                  ctypes.byref(c), None, s) == 0
    # the same update with its slots derived on the device: the same checks,
    # and a null start_pos is rejected (T > 0)
    assert L.kvq_quant_scatter_kv_full(None, None, 1, 1, 2, 4, 64, 0, 0, 64, None, ctypes.byref(c),
                                       ctypes.byref(cv_other), None, s) == 2
    assert L.kvq_quant_scatter_kv_full(None, None, 1, 1, 2, 4, 64, 0, 0, 64, None, ctypes.byref(c),
                                       ctypes.byref(c), None, s) == 1
    assert L.kvq_quant_scatter_kv_full(None, None, 5, 1, 2, 4, 64, 0, 0, 64, None, ctypes.byref(c),
                                       ctypes.byref(c), None, s) == 3
    assert L.kvq_quant_scatter_kv_full(None, None, 1, 1, 2, 0, 64, 0, 0, 64, None, ctypes.byref(c),
                                       ctypes.byref(c), None, s) == 0
    # positions: window must be >= 1, T >= 0
    assert L.kvq_positions_with_sink(None, 4, 4, 0, None, None, None, s) == 2
    assert L.kvq_positions_ring(None, -1, 8, None, None, None, s) == 2
    assert L.kvq_positions_full(None, 4, 0, None, None, None, s) == 2
    assert L.kvq_positions_full(None, 4, 16, None, None, None, s) == 1
    assert L.kvq_build_mask(None, 0, None, 1, 0, 4, None, s) == 2
    # the cache must be exactly its sink plus its window
    assert L.kvq_build_mask(None, 16, None, 1, 4, 8, None, s) == 2
    assert L.kvq_build_mask(None, 16, None, 1, 0, 17, None, s) == 2
    assert L.kvq_build_mask(None, 12, None, 0, 4, 8, None, s) == 0
    # block-mode caches pass validation (decode stops at the missing workspace)
    cb, keep3 = _fake_cache(kvq, qmode=kvq.FP8E4M3_B32, zps=False)
    q = ctypes.c_void_p(c.codes)
    assert L.kvq_sdpa_decode(q, 1, 1, 4, ctypes.byref(cb), ctypes.byref(cb), None, None, 0, 0, 0.1, q, 1,
                             None, 0, None, s) == 5
    # block-mode prefill with an unsupported head_dim is still rejected
    cb96, keep6 = _fake_cache(kvq, qmode=kvq.MXFP4_B32, D=96, zps=False)
    assert L.kvq_sdpa_prefill(q, 1, 1, 4, 8, ctypes.byref(cb96), ctypes.byref(cb96), None, None, 1, 0, 0.1, q, 1,
                              None, s) == 4
    # K and V caches in different modes
    assert L.kvq_sdpa_decode(q, 1, 1, 4, ctypes.byref(c), ctypes.byref(cb), None, None, 0, 0, 0.1, q, 1,
                             None, 0, None, s) == 3
    # per-batch lengths are required by the varlen entry points
    assert L.kvq_sdpa_decode_varlen(q, 1, 1, 4, ctypes.byref(c), ctypes.byref(c), None, None, 0, 0.1, q, 1,
                                    None, 0, None, s) == 1
    assert L.kvq_sdpa_prefill_varlen(q, 1, 1, 4, 8, ctypes.byref(c), ctypes.byref(c), None, None, 1, 0, 0.1, q, 1,
                                     None, s) == 1
    # Hq not a multiple of the KV heads
    assert L.kvq_sdpa_decode(q, 1, 1, 3, ctypes.byref(c), ctypes.byref(c), None, None, 0, 0, 0.1, q, 1,
                             None, 0, None, s) == 2
    # missing workspace
    assert L.kvq_sdpa_decode(q, 1, 1, 4, ctypes.byref(c), ctypes.byref(c), None, None, 0, 0, 0.1, q, 1,
                             None, 0, None, s) == 5
    # unsupported head_dim for attention
    c96, keep4 = _fake_cache(kvq, D=96)
    assert L.kvq_sdpa_prefill(q, 1, 1, 4, 8, ctypes.byref(c96), ctypes.byref(c96), None, None, 1, 0, 0.1, q, 1,
                              None, s) == 4
    # unknown prefill flag
    assert L.kvq_sdpa_prefill(q, 1, 1, 4, 8, ctypes.byref(c), ctypes.byref(c), None, None, 1, 2, 0.1, q, 1,
                              None, s) == 4
    # Lq beyond the cache
    assert L.kvq_sdpa_prefill(q, 1, 1, 4, 65, ctypes.byref(c), ctypes.byref(c), None, None, 1, 0, 0.1, q, 1,
                              None, s) == 2


def test_workspace_size(kvq):
    """A counter region (one 4-byte ticket per (b, kv head), rounded up to
    256 bytes) followed by whole per-split partials of (D + 2) fp32 values
    per (b, query head)."""
    n = kvq.sdpa_decode_workspace_bytes(8, 32, 8, 8192, 128)
    ctr = -(-8 * 8 * 4 // 256) * 256
    assert n > ctr and (n - ctr) % (8 * 32 * 130 * 4) == 0
    assert kvq.sdpa_decode_workspace_bytes(0, 32, 8, 8192, 128) == 0


def test_prefill_split_workspace(kvq):
    """Key-split prefill: the workspace size follows the sizes only (0 when the
    query tiles fill the part), and a missing or short workspace is rejected
    before anything is enqueued."""
    n = kvq.sdpa_prefill_split_workspace_bytes(1, 32, 8, 64, 16384, 128)
    assert n > 0 and n % (1 * 32 * 64 * 130 * 4) == 0
    assert kvq.sdpa_prefill_split_workspace_bytes(1, 32, 16, 2048, 131072, 256) == 0
    assert kvq.sdpa_prefill_split_workspace_bytes(1, 4, 2, 16, 256, 64) == 0      # too few keys to split
    assert kvq.sdpa_prefill_split_workspace_bytes(0, 32, 8, 64, 16384, 128) == 0
    assert kvq.sdpa_prefill_split_workspace_bytes(1, 30, 8, 64, 16384, 128) == 0  # Hq % heads != 0
    L = kvq.lib()
    c, keep = _fake_cache(kvq, S=4096)
    q = ctypes.c_void_p(c.codes)
    need = kvq.sdpa_prefill_split_workspace_bytes(1, 4, 2, 8, 4096, 64)
    assert need > 0
    assert L.kvq_sdpa_prefill_split(q, 1, 1, 4, 8, ctypes.byref(c), ctypes.byref(c), None, None, 1, 0, 0.1, q, 1,
                                    None, 0, None, None) == 5
    assert L.kvq_sdpa_prefill_split(q, 1, 1, 4, 8, ctypes.byref(c), ctypes.byref(c), None, None, 1, 0, 0.1, q, 1,
                                    q, need - 4, None, None) == 5
    assert L.kvq_sdpa_prefill_split_varlen(q, 1, 1, 4, 8, ctypes.byref(c), ctypes.byref(c), None, None, 1, 0, 0.1,
                                           q, 1, q, need, None, None) == 1      # kv_lens required
    # the ordinary argument checks come first
    assert L.kvq_sdpa_prefill_split(q, 1, 1, 3, 8, ctypes.byref(c), ctypes.byref(c), None, None, 1, 0, 0.1, q, 1,
                                    None, 0, None, None) == 2


def test_decode_append_full_validation(kvq):
    """kvq_sdpa_decode_append_full rejects on the host, nothing enqueued: null
    new rows or start_pos, a bad x dtype or stride, caches the single-pass
    int8 kernel does not take, shape errors as kvq_sdpa_decode, and a missing
    workspace."""
    L = kvq.lib()
    c, keep = _fake_cache(kvq)
    q = ctypes.c_void_p(c.codes)
    s = None

    def call(k=c, Hq=4, xk=q, xv=q, xd=1, xsb=128, xsh=64, sp=q, ws=None, wsb=0):
        return L.kvq_sdpa_decode_append_full(q, 1, 1, Hq, xk, xv, xd, xsb, xsh, sp, ctypes.byref(k), ctypes.byref(k),
                                             0.1, q, 1, ws, wsb, None, s)

    assert call(xk=None) == 1
    assert call(xv=None) == 1
    assert call(sp=None) == 1
    assert call(xd=5) == 3
    assert call(xsb=-1) == 2
    assert call(Hq=3) == 2
    c4, keep2 = _fake_cache(kvq, qmode=kvq.UINT4_TH)
    assert call(k=c4) == 4
    cb, keep3 = _fake_cache(kvq, qmode=kvq.FP8E4M3_B32, zps=False)
    assert call(k=cb) == 4
    c62, keep4 = _fake_cache(kvq, S=62)
    assert call(k=c62) == 4
    assert call() == 5


def test_decode_append_sink_validation(kvq):
    """kvq_sdpa_decode_append_sink: a null cache_positions, a layout that is
    not sink + window == n_slots, and the append checks of the full-context
    form, all on the host."""
    L = kvq.lib()
    c, keep = _fake_cache(kvq)                      # n_slots 64
    q = ctypes.c_void_p(c.codes)
    s = None

    def call(sink=4, window=60, cp=q, k=c, xk=q, Hq=4):
        return L.kvq_sdpa_decode_append_sink(q, 1, 1, Hq, xk, q, 1, 128, 64, q, sink, window, cp, ctypes.byref(k),
                                             ctypes.byref(k), 0.1, q, 1, None, 0, None, s)

    assert call(cp=None) == 1
    assert call(window=59) == 2
    assert call(sink=-1, window=65) == 2
    assert call(sink=64, window=0) == 2
    assert call(xk=None) == 1
    assert call(Hq=3) == 2
    c4, keep2 = _fake_cache(kvq, qmode=kvq.UINT4_TH)
    assert call(k=c4) == 4
    assert call() == 5
    assert call(sink=0, window=64) == 5
