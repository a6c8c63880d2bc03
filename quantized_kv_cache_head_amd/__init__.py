"""quantized_kv_cache_head_amd -- quantized KV cache write and attention on MI355X.

Thin Python binding of the C-ABI library ``libkvq.so`` (declared in
``include/kvq.h``).  Each function has the name of its C entry point without
the ``kvq_`` prefix and only marshals arguments: tensors become device
pointers, the current torch HIP stream is passed along, and a non-OK status
raises.  Every step runs in the library's HIP kernels; there is no CPU or
PyTorch fallback, and calling anything without the built library raises.

Build the library with ``python -m quantized_kv_cache_head_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

# kvq_qmode
INT8_TH, UINT4_TH, FP8E4M3_B32, MXFP4_B32 = 0, 1, 2, 3
MXFP8_B32, FP8E5M2_B32, INT8_B32, MXFP4E1M2_B32 = 4, 5, 6, 7
QMODES = {"int8": INT8_TH, "uint4": UINT4_TH, "fp8": FP8E4M3_B32, "mxfp4": MXFP4_B32, "mxfp8": MXFP8_B32,
          "fp8e5m2": FP8E5M2_B32, "int8_block": INT8_B32, "mxfp4_e1m2": MXFP4E1M2_B32}
BLOCK_MODES = (FP8E4M3_B32, MXFP4_B32, MXFP8_B32, FP8E5M2_B32, INT8_B32, MXFP4E1M2_B32)
E8M0_MODES = (MXFP4_B32, MXFP8_B32, MXFP4E1M2_B32)
# quantize options
MX_SCALE_OCP = 1
# kvq_dtype
F32, BF16 = 0, 1
# device error flags
FLAG_SLOT_RANGE, FLAG_KVLEN, FLAG_POS_CAPACITY = 1, 2, 4
NO_CAUSAL_SKIP = 1

EXPORTS = (
    "kvq_status_string", "kvq_cache_bytes", "kvq_quant_scatter", "kvq_quant_scatter_flags", "kvq_quant_scatter_kv",
    "kvq_quant_scatter_kv_full", "kvq_positions_with_sink",
    "kvq_positions_ring", "kvq_positions_full", "kvq_build_mask",
    "kvq_sdpa_decode_workspace_bytes", "kvq_sdpa_decode", "kvq_sdpa_decode_varlen", "kvq_sdpa_prefill",
    "kvq_sdpa_prefill_varlen", "kvq_sdpa_prefill_split_workspace_bytes", "kvq_sdpa_prefill_split",
    "kvq_sdpa_prefill_split_varlen", "kvq_sdpa_decode_noalloc", "kvq_sdpa_decode_append_full",
    "kvq_sdpa_decode_append_sink",
)


class KvqError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


class kvq_cache(ctypes.Structure):
    _fields_ = [("qmode", ctypes.c_int32), ("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("n_slots", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("zps", ctypes.c_void_p)]


_lib = None
_P, _I, _I64, _SZ, _F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
_CP = ctypes.POINTER(kvq_cache)


def lib():
    """The loaded libkvq.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m quantized_kv_cache_head_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.kvq_status_string.restype = ctypes.c_char_p
        L.kvq_status_string.argtypes = [_I]
        L.kvq_cache_bytes.restype = _I
        L.kvq_cache_bytes.argtypes = [_I, _I, _I, _I, _I, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]
        L.kvq_quant_scatter.restype = _I
        L.kvq_quant_scatter.argtypes = [_P, _I, _I, _I, _I, _I, _I64, _I64, _I64, _P, _I64, _CP, _P, _P]
        L.kvq_quant_scatter_flags.restype = _I
        L.kvq_quant_scatter_flags.argtypes = [_P, _I, _I, _I, _I, _I, _I64, _I64, _I64, _P, _I64, _CP, ctypes.c_uint,
                                              _P, _P]
        L.kvq_quant_scatter_kv.restype = _I
        L.kvq_quant_scatter_kv.argtypes = [_P, _P, _I, _I, _I, _I, _I, _I64, _I64, _I64, _P, _I64, _CP, _CP, _P, _P]
        L.kvq_quant_scatter_kv_full.restype = _I
        L.kvq_quant_scatter_kv_full.argtypes = [_P, _P, _I, _I, _I, _I, _I, _I64, _I64, _I64, _P, _CP, _CP, _P, _P]
        L.kvq_positions_with_sink.restype = _I
        L.kvq_positions_with_sink.argtypes = [_P, _I, _I, _I, _P, _P, _P, _P]
        L.kvq_positions_ring.restype = _I
        L.kvq_positions_ring.argtypes = [_P, _I, _I, _P, _P, _P, _P]
        L.kvq_positions_full.restype = _I
        L.kvq_positions_full.argtypes = [_P, _I, _I, _P, _P, _P, _P]
        L.kvq_build_mask.restype = _I
        L.kvq_build_mask.argtypes = [_P, _I, _P, _I, _I, _I, _P, _P]
        L.kvq_sdpa_decode_workspace_bytes.restype = _SZ
        L.kvq_sdpa_decode_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
        L.kvq_sdpa_decode.restype = _I
        L.kvq_sdpa_decode.argtypes = [_P, _I, _I, _I, _CP, _CP, _P, _P, _I64, _I, _F, _P, _I, _P, _SZ, _P, _P]
        L.kvq_sdpa_decode_append_full.restype = _I
        L.kvq_sdpa_decode_append_full.argtypes = [_P, _I, _I, _I, _P, _P, _I, _I64, _I64, _P, _CP, _CP, _F, _P, _I,
                                                  _P, _SZ, _P, _P]
        L.kvq_sdpa_decode_append_sink.restype = _I
        L.kvq_sdpa_decode_append_sink.argtypes = [_P, _I, _I, _I, _P, _P, _I, _I64, _I64, _P, _I, _I, _P, _CP, _CP, _F,
                                                  _P, _I, _P, _SZ, _P, _P]
        L.kvq_sdpa_decode_noalloc.restype = _I
        L.kvq_sdpa_decode_noalloc.argtypes = [_P, _I, _I, _I, _CP, _CP, _P, _P, _I64, _I, _F, _P, _I, _P, _P]
        L.kvq_sdpa_prefill.restype = _I
        L.kvq_sdpa_prefill.argtypes = [_P, _I, _I, _I, _I, _CP, _CP, _P, _P, _I, ctypes.c_uint, _F, _P, _I, _P, _P]
        L.kvq_sdpa_decode_varlen.restype = _I
        L.kvq_sdpa_decode_varlen.argtypes = [_P, _I, _I, _I, _CP, _CP, _P, _P, _I64, _F, _P, _I, _P, _SZ, _P, _P]
        L.kvq_sdpa_prefill_varlen.restype = _I
        L.kvq_sdpa_prefill_varlen.argtypes = [_P, _I, _I, _I, _I, _CP, _CP, _P, _P, _I, ctypes.c_uint, _F, _P, _I,
                                              _P, _P]
        L.kvq_sdpa_prefill_split_workspace_bytes.restype = _SZ
        L.kvq_sdpa_prefill_split_workspace_bytes.argtypes = [_I, _I, _I, _I, _I, _I]
        L.kvq_sdpa_prefill_split.restype = _I
        L.kvq_sdpa_prefill_split.argtypes = [_P, _I, _I, _I, _I, _CP, _CP, _P, _P, _I, ctypes.c_uint, _F, _P, _I,
                                             _P, _SZ, _P, _P]
        L.kvq_sdpa_prefill_split_varlen.restype = _I
        L.kvq_sdpa_prefill_split_varlen.argtypes = L.kvq_sdpa_prefill_split.argtypes
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().kvq_status_string(int(status)).decode()


def _check(fn, st):
    if st != 0:
        raise KvqError(fn, st)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


# --------------------------------------------------------------------------
# Cache planes
# --------------------------------------------------------------------------

def cache_bytes(qmode: int, B: int, H: int, n_slots: int, D: int):
    c, s, z = _SZ(), _SZ(), _SZ()
    _check("kvq_cache_bytes", lib().kvq_cache_bytes(qmode, B, H, n_slots, D, ctypes.byref(c), ctypes.byref(s), ctypes.byref(z)))
    return c.value, s.value, z.value


@dataclass
class Cache:
    """One quantized cache (K or V): caller-owned device planes.

    codes  uint8 [B, H, S, row_bytes]
    scales float32 [B, H, S, spr] (uint8 E8M0 for MX-FP4)
    zps    int8 [B, H, S] (affine modes) or None
    """
    qmode: int
    B: int
    H: int
    S: int
    D: int
    codes: torch.Tensor
    scales: torch.Tensor
    zps: torch.Tensor | None

    @staticmethod
    def empty(qmode, B, H, S, D, device="cuda"):
        cb, sb, zb = cache_bytes(qmode, B, H, S, D)
        rb = cb // (B * H * S)
        spr = (D // 32) if qmode in BLOCK_MODES else 1
        codes = torch.empty((B, H, S, rb), dtype=torch.uint8, device=device)
        sdt = torch.uint8 if qmode in E8M0_MODES else torch.float32
        scales = torch.empty((B, H, S, spr), dtype=sdt, device=device)
        zps = torch.empty((B, H, S), dtype=torch.int8, device=device) if zb else None
        return Cache(qmode, B, H, S, D, codes, scales, zps)

    def sentinel_fill(self):
        """Codes 0xA5, scales NaN (0xFF for E8M0), zero points 0x5A."""
        self.codes.fill_(0xA5)
        if self.scales.dtype == torch.uint8:
            self.scales.fill_(0xFF)
        else:
            self.scales.fill_(float("nan"))
        if self.zps is not None:
            self.zps.fill_(0x5A)
        return self

    def struct(self) -> kvq_cache:
        return kvq_cache(self.qmode, self.B, self.H, self.S, self.D, self.codes.data_ptr(),
                         self.scales.data_ptr(), 0 if self.zps is None else self.zps.data_ptr())

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.codes, self.scales, self.zps) if t is not None)


# --------------------------------------------------------------------------
# Entry points
# --------------------------------------------------------------------------

def quant_scatter(x: torch.Tensor, slot_mapping: torch.Tensor, cache: Cache, err_flags=None, stream=None, flags=0):
    """kvq_quant_scatter (kvq_quant_scatter_flags when flags != 0): x [B, H, T, D]
    (bf16/fp32, D contiguous); slot_mapping int32 [B, T] or [T] (shared over
    the batch); flags: MX_SCALE_OCP for the MX modes."""
    _need_cuda(x, slot_mapping, err_flags)
    if x.dim() != 4 or x.stride(3) != 1:
        raise ValueError("x must be [B, H, T, D] with D contiguous")
    if slot_mapping.dtype != torch.int32 or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be contiguous int32")
    B, H, T, D = x.shape
    ssb = 0 if slot_mapping.dim() == 1 else slot_mapping.stride(0)
    c = cache.struct()
    if flags:
        _check("kvq_quant_scatter_flags", lib().kvq_quant_scatter_flags(
            _ptr(x), _dtype_code(x), B, H, T, D, x.stride(0), x.stride(1), x.stride(2),
            _ptr(slot_mapping), ssb, ctypes.byref(c), int(flags), _ptr(err_flags), _stream(stream)))
        return
    _check("kvq_quant_scatter", lib().kvq_quant_scatter(
        _ptr(x), _dtype_code(x), B, H, T, D, x.stride(0), x.stride(1), x.stride(2),
        _ptr(slot_mapping), ssb, ctypes.byref(c), _ptr(err_flags), _stream(stream)))


def quant_scatter_kv(xk: torch.Tensor, xv: torch.Tensor, slot_mapping: torch.Tensor, k_cache: Cache, v_cache: Cache,
                     err_flags=None, stream=None):
    """kvq_quant_scatter_kv: the K and V update of one step in one launch; xk and
    xv are [B, H, T, D] with the same dtype, shape and strides."""
    _need_cuda(xk, xv, slot_mapping, err_flags)
    if xk.dim() != 4 or xk.stride(3) != 1 or xk.shape != xv.shape or xk.stride() != xv.stride() or xk.dtype != xv.dtype:
        raise ValueError("xk and xv must be [B, H, T, D] with D contiguous, equal shapes, strides and dtype")
    if slot_mapping.dtype != torch.int32 or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be contiguous int32")
    B, H, T, D = xk.shape
    ssb = 0 if slot_mapping.dim() == 1 else slot_mapping.stride(0)
    kc, vc = k_cache.struct(), v_cache.struct()
    _check("kvq_quant_scatter_kv", lib().kvq_quant_scatter_kv(
        _ptr(xk), _ptr(xv), _dtype_code(xk), B, H, T, D, xk.stride(0), xk.stride(1), xk.stride(2),
        _ptr(slot_mapping), ssb, ctypes.byref(kc), ctypes.byref(vc), _ptr(err_flags), _stream(stream)))


def quant_scatter_kv_full(xk: torch.Tensor, xv: torch.Tensor, start_pos: torch.Tensor, k_cache: Cache,
                          v_cache: Cache, err_flags=None, stream=None):
    """kvq_quant_scatter_kv_full: positions_full and quant_scatter_kv in one
    launch (token t to slot *start_pos + t); start_pos a device int32 scalar."""
    _need_cuda(xk, xv, start_pos, err_flags)
    if xk.dim() != 4 or xk.stride(3) != 1 or xk.shape != xv.shape or xk.stride() != xv.stride() or xk.dtype != xv.dtype:
        raise ValueError("xk and xv must be [B, H, T, D] with D contiguous, equal shapes, strides and dtype")
    if start_pos.dtype != torch.int32 or start_pos.numel() != 1:
        raise ValueError("start_pos must be one int32")
    B, H, T, D = xk.shape
    kc, vc = k_cache.struct(), v_cache.struct()
    _check("kvq_quant_scatter_kv_full", lib().kvq_quant_scatter_kv_full(
        _ptr(xk), _ptr(xv), _dtype_code(xk), B, H, T, D, xk.stride(0), xk.stride(1), xk.stride(2),
        _ptr(start_pos), ctypes.byref(kc), ctypes.byref(vc), _ptr(err_flags), _stream(stream)))


def positions_with_sink(start_pos, T, sink_size, window, slot_mapping_out, cache_positions, err_flags=None, stream=None):
    _need_cuda(start_pos, slot_mapping_out, cache_positions, err_flags)
    _check("kvq_positions_with_sink", lib().kvq_positions_with_sink(
        _ptr(start_pos), T, sink_size, window, _ptr(slot_mapping_out), _ptr(cache_positions),
        _ptr(err_flags), _stream(stream)))


def positions_ring(start_pos, T, window, slot_mapping_out, cache_positions, err_flags=None, stream=None):
    _need_cuda(start_pos, slot_mapping_out, cache_positions, err_flags)
    _check("kvq_positions_ring", lib().kvq_positions_ring(
        _ptr(start_pos), T, window, _ptr(slot_mapping_out), _ptr(cache_positions), _ptr(err_flags), _stream(stream)))


def positions_full(start_pos, T, capacity, slot_mapping_out, cache_positions=None, err_flags=None, stream=None):
    _need_cuda(start_pos, slot_mapping_out, cache_positions, err_flags)
    _check("kvq_positions_full", lib().kvq_positions_full(
        _ptr(start_pos), T, capacity, _ptr(slot_mapping_out), _ptr(cache_positions), _ptr(err_flags), _stream(stream)))


def build_mask(cache_positions, start_pos, Lq, sink_size, window, mask_out, stream=None):
    _need_cuda(cache_positions, start_pos, mask_out)
    n_slots = cache_positions.numel()
    if mask_out.dtype != torch.float32 or mask_out.numel() != Lq * n_slots:
        raise ValueError("mask_out must be float32 [Lq, n_slots]")
    _check("kvq_build_mask", lib().kvq_build_mask(
        _ptr(cache_positions), n_slots, _ptr(start_pos), Lq, sink_size, window, _ptr(mask_out), _stream(stream)))


def sdpa_decode_workspace_bytes(B, Hq, Hkv, n_slots, D) -> int:
    return int(lib().kvq_sdpa_decode_workspace_bytes(B, Hq, Hkv, n_slots, D))


def decode_workspace(B, Hq, Hkv, n_slots, D, device="cuda"):
    """A workspace for sdpa_decode (per-split partial results)."""
    return torch.zeros(sdpa_decode_workspace_bytes(B, Hq, Hkv, n_slots, D), dtype=torch.uint8, device=device)


def sdpa_decode(q, k: Cache, v: Cache, kv_len=None, mask=None, sm_scale=None, out=None,
                out_dtype=None, workspace=None, err_flags=None, mask_is_causal=False, stream=None):
    """kvq_sdpa_decode: q [B, Hq, 1, D]; returns out [B, Hq, 1, D]."""
    _need_cuda(q, kv_len, mask, out, workspace, err_flags)
    B, Hq, Lq, D = q.shape
    if Lq != 1 or not q.is_contiguous():
        raise ValueError("q must be contiguous [B, Hq, 1, D]")
    if sm_scale is None:
        sm_scale = D ** -0.5
    if out is None:
        out = torch.empty((B, Hq, 1, D), dtype=out_dtype or q.dtype, device=q.device)
    if workspace is None:
        workspace = decode_workspace(B, Hq, k.H, k.S, D, q.device)
    msb = 0
    if mask is not None:
        if mask.dtype != torch.float32 or not mask.is_contiguous():
            raise ValueError("mask must be contiguous float32 [n_slots] or [B, n_slots]")
        msb = 0 if mask.dim() == 1 or mask.shape[0] == 1 else mask.stride(0)
    kc, vc = k.struct(), v.struct()
    _check("kvq_sdpa_decode", lib().kvq_sdpa_decode(
        _ptr(q), _dtype_code(q), B, Hq, ctypes.byref(kc), ctypes.byref(vc), _ptr(kv_len), _ptr(mask), msb,
        int(bool(mask_is_causal)), float(sm_scale), _ptr(out), _dtype_code(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(err_flags), _stream(stream)))
    return out


def sdpa_decode_append_full(q, xk, xv, start_pos, k: Cache, v: Cache, sm_scale=None, out=None, out_dtype=None,
                            workspace=None, err_flags=None, stream=None):
    """kvq_sdpa_decode_append_full: the new token's K and V (xk, xv [B, Hkv, 1,
    D], D contiguous) written at slot *start_pos of full-context caches, then
    decode attention of q [B, Hq, 1, D] over kv_len = *start_pos + 1, in one
    launch; returns out [B, Hq, 1, D]."""
    _need_cuda(q, xk, xv, start_pos, out, workspace, err_flags)
    B, Hq, Lq, D = q.shape
    if Lq != 1 or not q.is_contiguous():
        raise ValueError("q must be contiguous [B, Hq, 1, D]")
    if (xk.dim() != 4 or xk.shape != xv.shape or xk.shape[2] != 1 or xk.stride(3) != 1 or xv.stride(3) != 1
            or xk.stride()[:2] != xv.stride()[:2] or xk.dtype != xv.dtype):
        raise ValueError("xk and xv must be [B, Hkv, 1, D] with D contiguous, equal shapes, strides and dtype")
    if start_pos.dtype != torch.int32 or start_pos.numel() != 1:
        raise ValueError("start_pos must be one int32")
    if sm_scale is None:
        sm_scale = D ** -0.5
    if out is None:
        out = torch.empty((B, Hq, 1, D), dtype=out_dtype or q.dtype, device=q.device)
    if workspace is None:
        workspace = decode_workspace(B, Hq, k.H, k.S, D, q.device)
    kc, vc = k.struct(), v.struct()
    _check("kvq_sdpa_decode_append_full", lib().kvq_sdpa_decode_append_full(
        _ptr(q), _dtype_code(q), B, Hq, _ptr(xk), _ptr(xv), _dtype_code(xk), xk.stride(0), xk.stride(1),
        _ptr(start_pos), ctypes.byref(kc), ctypes.byref(vc), float(sm_scale), _ptr(out), _dtype_code(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(err_flags), _stream(stream)))
    return out


def sdpa_decode_append_sink(q, xk, xv, start_pos, sink_size, window, cache_positions, k: Cache, v: Cache,
                            sm_scale=None, out=None, out_dtype=None, workspace=None, err_flags=None, stream=None):
    """kvq_sdpa_decode_append_sink: the sink / ring form of
    sdpa_decode_append_full (slot from the positions manager with sink,
    cache_positions int32 [n_slots] updated, keys masked by the additive-mask
    rule); returns out [B, Hq, 1, D]."""
    _need_cuda(q, xk, xv, start_pos, cache_positions, out, workspace, err_flags)
    B, Hq, Lq, D = q.shape
    if Lq != 1 or not q.is_contiguous():
        raise ValueError("q must be contiguous [B, Hq, 1, D]")
    if (xk.dim() != 4 or xk.shape != xv.shape or xk.shape[2] != 1 or xk.stride(3) != 1 or xv.stride(3) != 1
            or xk.stride()[:2] != xv.stride()[:2] or xk.dtype != xv.dtype):
        raise ValueError("xk and xv must be [B, Hkv, 1, D] with D contiguous, equal shapes, strides and dtype")
    if start_pos.dtype != torch.int32 or start_pos.numel() != 1:
        raise ValueError("start_pos must be one int32")
    if cache_positions.dtype != torch.int32 or not cache_positions.is_contiguous():
        raise ValueError("cache_positions must be contiguous int32 [n_slots]")
    if sm_scale is None:
        sm_scale = D ** -0.5
    if out is None:
        out = torch.empty((B, Hq, 1, D), dtype=out_dtype or q.dtype, device=q.device)
    if workspace is None:
        workspace = decode_workspace(B, Hq, k.H, k.S, D, q.device)
    kc, vc = k.struct(), v.struct()
    _check("kvq_sdpa_decode_append_sink", lib().kvq_sdpa_decode_append_sink(
        _ptr(q), _dtype_code(q), B, Hq, _ptr(xk), _ptr(xv), _dtype_code(xk), xk.stride(0), xk.stride(1),
        _ptr(start_pos), int(sink_size), int(window), _ptr(cache_positions), ctypes.byref(kc), ctypes.byref(vc),
        float(sm_scale), _ptr(out), _dtype_code(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(err_flags), _stream(stream)))
    return out


def sdpa_decode_noalloc(q, k: Cache, v: Cache, kv_len=None, mask=None, sm_scale=None, out=None,
                        out_dtype=None, err_flags=None, mask_is_causal=False, stream=None):
    """kvq_sdpa_decode_noalloc: kvq_sdpa_decode on the library's own per-GPU
    scratch array (no workspace); allocates only `out` when it is None."""
    _need_cuda(q, kv_len, mask, out, err_flags)
    B, Hq, Lq, D = q.shape
    if Lq != 1 or not q.is_contiguous():
        raise ValueError("q must be contiguous [B, Hq, 1, D]")
    if sm_scale is None:
        sm_scale = D ** -0.5
    if out is None:
        out = torch.empty((B, Hq, 1, D), dtype=out_dtype or q.dtype, device=q.device)
    msb = 0
    if mask is not None:
        if mask.dtype != torch.float32 or not mask.is_contiguous():
            raise ValueError("mask must be contiguous float32 [n_slots] or [B, n_slots]")
        msb = 0 if mask.dim() == 1 or mask.shape[0] == 1 else mask.stride(0)
    kc, vc = k.struct(), v.struct()
    _check("kvq_sdpa_decode_noalloc", lib().kvq_sdpa_decode_noalloc(
        _ptr(q), _dtype_code(q), B, Hq, ctypes.byref(kc), ctypes.byref(vc), _ptr(kv_len), _ptr(mask), msb,
        int(bool(mask_is_causal)), float(sm_scale), _ptr(out), _dtype_code(out), _ptr(err_flags),
        _stream(stream)))
    return out


def sdpa_prefill(q, k: Cache, v: Cache, kv_len=None, mask=None, causal=True, sm_scale=None, out=None,
                 out_dtype=None, no_causal_skip=False, err_flags=None, stream=None):
    """kvq_sdpa_prefill: q [B, Hq, Lq, D] at positions [kv_len - Lq, kv_len)."""
    _need_cuda(q, kv_len, mask, out, err_flags)
    B, Hq, Lq, D = q.shape
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if sm_scale is None:
        sm_scale = D ** -0.5
    if out is None:
        out = torch.empty((B, Hq, Lq, D), dtype=out_dtype or q.dtype, device=q.device)
    if mask is not None and (mask.dtype != torch.float32 or not mask.is_contiguous()):
        raise ValueError("mask must be contiguous float32 [Lq, n_slots]")
    kc, vc = k.struct(), v.struct()
    _check("kvq_sdpa_prefill", lib().kvq_sdpa_prefill(
        _ptr(q), _dtype_code(q), B, Hq, Lq, ctypes.byref(kc), ctypes.byref(vc), _ptr(kv_len), _ptr(mask),
        int(bool(causal)), NO_CAUSAL_SKIP if no_causal_skip else 0, float(sm_scale), _ptr(out),
        _dtype_code(out), _ptr(err_flags), _stream(stream)))
    return out


def sdpa_prefill_split_workspace_bytes(B, Hq, Hkv, Lq, n_slots, D) -> int:
    return int(lib().kvq_sdpa_prefill_split_workspace_bytes(B, Hq, Hkv, Lq, n_slots, D))


def sdpa_prefill_split(q, k: Cache, v: Cache, kv_len=None, mask=None, causal=True, sm_scale=None, out=None,
                       out_dtype=None, no_causal_skip=False, workspace=None, err_flags=None, stream=None):
    """kvq_sdpa_prefill_split: sdpa_prefill with each query tile's key range split
    over several workgroups, for short chunks; workspace as sized by
    sdpa_prefill_split_workspace_bytes (allocated here when None)."""
    _need_cuda(q, kv_len, mask, out, workspace, err_flags)
    B, Hq, Lq, D = q.shape
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if sm_scale is None:
        sm_scale = D ** -0.5
    if out is None:
        out = torch.empty((B, Hq, Lq, D), dtype=out_dtype or q.dtype, device=q.device)
    if mask is not None and (mask.dtype != torch.float32 or not mask.is_contiguous()):
        raise ValueError("mask must be contiguous float32 [Lq, n_slots]")
    if workspace is None:
        nb = sdpa_prefill_split_workspace_bytes(B, Hq, k.H, Lq, k.S, D)
        workspace = torch.empty(max(nb, 1), dtype=torch.uint8, device=q.device)
    kc, vc = k.struct(), v.struct()
    _check("kvq_sdpa_prefill_split", lib().kvq_sdpa_prefill_split(
        _ptr(q), _dtype_code(q), B, Hq, Lq, ctypes.byref(kc), ctypes.byref(vc), _ptr(kv_len), _ptr(mask),
        int(bool(causal)), NO_CAUSAL_SKIP if no_causal_skip else 0, float(sm_scale), _ptr(out),
        _dtype_code(out), _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(err_flags),
        _stream(stream)))
    return out


def sdpa_prefill_split_varlen(q, k: Cache, v: Cache, kv_lens, mask=None, causal=True, sm_scale=None, out=None,
                              out_dtype=None, no_causal_skip=False, workspace=None, err_flags=None, stream=None):
    """kvq_sdpa_prefill_split_varlen: sdpa_prefill_split with kv_lens int32 [B] on the device."""
    _need_cuda(q, kv_lens, mask, out, workspace, err_flags)
    B, Hq, Lq, D = q.shape
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if kv_lens.dtype != torch.int32 or kv_lens.numel() != B or not kv_lens.is_contiguous():
        raise ValueError("kv_lens must be contiguous int32 [B]")
    if sm_scale is None:
        sm_scale = D ** -0.5
    if out is None:
        out = torch.empty((B, Hq, Lq, D), dtype=out_dtype or q.dtype, device=q.device)
    if mask is not None and (mask.dtype != torch.float32 or not mask.is_contiguous()):
        raise ValueError("mask must be contiguous float32 [Lq, n_slots]")
    if workspace is None:
        nb = sdpa_prefill_split_workspace_bytes(B, Hq, k.H, Lq, k.S, D)
        workspace = torch.empty(max(nb, 1), dtype=torch.uint8, device=q.device)
    kc, vc = k.struct(), v.struct()
    _check("kvq_sdpa_prefill_split_varlen", lib().kvq_sdpa_prefill_split_varlen(
        _ptr(q), _dtype_code(q), B, Hq, Lq, ctypes.byref(kc), ctypes.byref(vc), _ptr(kv_lens), _ptr(mask),
        int(bool(causal)), NO_CAUSAL_SKIP if no_causal_skip else 0, float(sm_scale), _ptr(out),
        _dtype_code(out), _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(err_flags),
        _stream(stream)))
    return out


def sdpa_decode_varlen(q, k: Cache, v: Cache, kv_lens, mask=None, sm_scale=None, out=None, out_dtype=None,
                       workspace=None, err_flags=None, stream=None):
    """kvq_sdpa_decode_varlen: as sdpa_decode with kv_lens int32 [B] on the device."""
    _need_cuda(q, kv_lens, mask, out, workspace, err_flags)
    B, Hq, Lq, D = q.shape
    if Lq != 1 or not q.is_contiguous():
        raise ValueError("q must be contiguous [B, Hq, 1, D]")
    if kv_lens.dtype != torch.int32 or kv_lens.numel() != B or not kv_lens.is_contiguous():
        raise ValueError("kv_lens must be contiguous int32 [B]")
    if sm_scale is None:
        sm_scale = D ** -0.5
    if out is None:
        out = torch.empty((B, Hq, 1, D), dtype=out_dtype or q.dtype, device=q.device)
    if workspace is None:
        workspace = decode_workspace(B, Hq, k.H, k.S, D, q.device)
    msb = 0
    if mask is not None:
        if mask.dtype != torch.float32 or not mask.is_contiguous():
            raise ValueError("mask must be contiguous float32 [n_slots] or [B, n_slots]")
        msb = 0 if mask.dim() == 1 or mask.shape[0] == 1 else mask.stride(0)
    kc, vc = k.struct(), v.struct()
    _check("kvq_sdpa_decode_varlen", lib().kvq_sdpa_decode_varlen(
        _ptr(q), _dtype_code(q), B, Hq, ctypes.byref(kc), ctypes.byref(vc), _ptr(kv_lens), _ptr(mask), msb,
        float(sm_scale), _ptr(out), _dtype_code(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(err_flags), _stream(stream)))
    return out


def sdpa_prefill_varlen(q, k: Cache, v: Cache, kv_lens, mask=None, causal=True, sm_scale=None, out=None,
                        out_dtype=None, no_causal_skip=False, err_flags=None, stream=None):
    """kvq_sdpa_prefill_varlen: as sdpa_prefill with kv_lens int32 [B] on the device."""
    _need_cuda(q, kv_lens, mask, out, err_flags)
    B, Hq, Lq, D = q.shape
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if kv_lens.dtype != torch.int32 or kv_lens.numel() != B or not kv_lens.is_contiguous():
        raise ValueError("kv_lens must be contiguous int32 [B]")
    if sm_scale is None:
        sm_scale = D ** -0.5
    if out is None:
        out = torch.empty((B, Hq, Lq, D), dtype=out_dtype or q.dtype, device=q.device)
    if mask is not None and (mask.dtype != torch.float32 or not mask.is_contiguous()):
        raise ValueError("mask must be contiguous float32 [Lq, n_slots]")
    kc, vc = k.struct(), v.struct()
    _check("kvq_sdpa_prefill_varlen", lib().kvq_sdpa_prefill_varlen(
        _ptr(q), _dtype_code(q), B, Hq, Lq, ctypes.byref(kc), ctypes.byref(vc), _ptr(kv_lens), _ptr(mask),
        int(bool(causal)), NO_CAUSAL_SKIP if no_causal_skip else 0, float(sm_scale), _ptr(out),
        _dtype_code(out), _ptr(err_flags), _stream(stream)))
    return out
