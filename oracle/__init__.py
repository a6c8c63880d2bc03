"""CPU oracle for the quantized KV-cache hot path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  The product library never loads it; the two share no code.

The arithmetic lives in ``kvq_oracle.c`` (plain scalar C, fp32 encode steps,
fp64 attention, ``-ffp-contract=off``); this module only compiles it with gcc
and marshals NumPy arrays through ctypes.  See the header of ``kvq_oracle.c``
for the passages of the pages each function follows and the readings taken
where they are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB = os.path.join(_HERE, "libkvq_oracle.so")

INT8_TH, UINT4_TH, FP8E4M3_B32, MXFP4_B32 = 0, 1, 2, 3
MXFP8_B32, FP8E5M2_B32, INT8_B32, MXFP4E1M2_B32 = 4, 5, 6, 7
BLOCK_MODES = (FP8E4M3_B32, MXFP4_B32, MXFP8_B32, FP8E5M2_B32, INT8_B32, MXFP4E1M2_B32)
E8M0_MODES = (MXFP4_B32, MXFP8_B32, MXFP4E1M2_B32)
MX_SCALE_OCP = 1            # quantize option: MX scale by the OCP floor rule
FLAG_SLOT_RANGE, FLAG_KVLEN, FLAG_POS_CAPACITY = 1, 2, 4

CFLAGS = ["-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-fPIC", "-shared", "-Wall"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/libkvq_oracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = ctypes.CDLL(_LIB)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I = ctypes.c_int
_LL = ctypes.c_longlong
_D = ctypes.c_double


def _declare(L):
    L.orc_e4m3fn_encode.restype = ctypes.c_uint8
    L.orc_e4m3fn_encode.argtypes = [ctypes.c_float]
    L.orc_e4m3fn_decode.restype = ctypes.c_float
    L.orc_e4m3fn_decode.argtypes = [ctypes.c_uint8]
    L.orc_e2m1_encode.restype = ctypes.c_uint8
    L.orc_e2m1_encode.argtypes = [ctypes.c_float]
    L.orc_e2m1_decode.restype = ctypes.c_float
    L.orc_e2m1_decode.argtypes = [ctypes.c_uint8]
    L.orc_e1m2_decode.restype = ctypes.c_float
    L.orc_e1m2_decode.argtypes = [ctypes.c_uint8]
    L.orc_e8m0_ceil.restype = ctypes.c_uint8
    L.orc_e8m0_ceil.argtypes = [ctypes.c_float]
    for name in ("orc_e4m3fn_encode_array", "orc_e2m1_encode_array", "orc_e8m0_ceil_array",
                 "orc_e5m2_encode_array", "orc_e1m2_encode_array"):
        f = getattr(L, name)
        f.restype = None
        f.argtypes = [_P, _P, _LL]
    L.orc_e5m2_decode.restype = ctypes.c_float
    L.orc_e5m2_decode.argtypes = [ctypes.c_uint8]
    L.orc_e8m0_floor_array.restype = None
    L.orc_e8m0_floor_array.argtypes = [_P, _I, _P, _LL]
    L.orc_affine_params.restype = None
    L.orc_affine_params.argtypes = [_P, _I, _I, _I, _P, _P]
    L.orc_quantize_rows.restype = None
    L.orc_quantize_rows.argtypes = [_I, _P, _I, _I, _P, _P, _P]
    L.orc_quantize_rows_f.restype = None
    L.orc_quantize_rows_f.argtypes = [_I, _I, _P, _I, _I, _P, _P, _P]
    L.orc_dequantize_rows.restype = None
    L.orc_dequantize_rows.argtypes = [_I, _P, _P, _P, _I, _I, _P]
    for name in ("orc_quant_scatter", "orc_quant_scatter_par"):
        f = getattr(L, name)
        f.restype = _I
        f.argtypes = [_I, _P, _I, _I, _I, _I, _P, _LL, _I, _P, _P, _P]
    for name in ("orc_quant_scatter_f", "orc_quant_scatter_par_f"):
        f = getattr(L, name)
        f.restype = _I
        f.argtypes = [_I, _I, _P, _I, _I, _I, _I, _P, _LL, _I, _P, _P, _P]
    L.orc_positions_sink.restype = _I
    L.orc_positions_sink.argtypes = [_I, _I, _I, _I, _P, _P]
    L.orc_positions_full.restype = _I
    L.orc_positions_full.argtypes = [_I, _I, _I, _P, _P]
    L.orc_build_mask.restype = None
    L.orc_build_mask.argtypes = [_P, _I, _I, _I, _I, _I, _P]
    L.orc_sdpa.restype = _I
    L.orc_sdpa.argtypes = [_P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P,
                           _I, _P, _LL, _I, _D, _P]
    L.orc_sdpa_rows.restype = _I
    L.orc_sdpa_rows.argtypes = [_P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P,
                                _I, _P, _LL, _I, _D, _P, _I, _P]


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    """Contiguous array of exactly ``dtype`` (no silent copies of caches)."""
    a = np.ascontiguousarray(a)
    if a.dtype != np.dtype(dtype):
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


# --------------------------------------------------------------------------
# Element encoders
# --------------------------------------------------------------------------

def e4m3fn_encode(y):
    y = _c(np.asarray(y, dtype=np.float32), np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().orc_e4m3fn_encode_array(_ptr(y), _ptr(out), y.size)
    return out


def e2m1_encode(y):
    y = _c(np.asarray(y, dtype=np.float32), np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().orc_e2m1_encode_array(_ptr(y), _ptr(out), y.size)
    return out


def e1m2_encode(y):
    y = _c(np.asarray(y, dtype=np.float32), np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().orc_e1m2_encode_array(_ptr(y), _ptr(out), y.size)
    return out


def e8m0_ceil(s):
    s = _c(np.asarray(s, dtype=np.float32), np.float32)
    out = np.empty(s.shape, np.uint8)
    lib().orc_e8m0_ceil_array(_ptr(s), _ptr(out), s.size)
    return out


def e5m2_encode(y):
    y = _c(np.asarray(y, dtype=np.float32), np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().orc_e5m2_encode_array(_ptr(y), _ptr(out), y.size)
    return out


def e8m0_floor(amax, emax: int):
    a = _c(np.asarray(amax, dtype=np.float32), np.float32)
    out = np.empty(a.shape, np.uint8)
    lib().orc_e8m0_floor_array(_ptr(a), int(emax), _ptr(out), a.size)
    return out


def e5m2_decode(code: int) -> float:
    return lib().orc_e5m2_decode(int(code))


def e4m3fn_decode(code: int) -> float:
    return lib().orc_e4m3fn_decode(int(code))


def e2m1_decode(code: int) -> float:
    return lib().orc_e2m1_decode(int(code))


def e1m2_decode(code: int) -> float:
    return lib().orc_e1m2_decode(int(code))


def affine_params(x, qmin: int, qmax: int):
    x = _c(np.asarray(x, dtype=np.float32), np.float32)
    scale = ctypes.c_float()
    zp = ctypes.c_int()
    lib().orc_affine_params(_ptr(x), x.size, qmin, qmax, ctypes.byref(scale), ctypes.byref(zp))
    return scale.value, zp.value


# --------------------------------------------------------------------------
# Cache geometry and containers
# --------------------------------------------------------------------------

def row_bytes(qmode: int, D: int) -> int:
    return D // 2 if qmode in (UINT4_TH, MXFP4_B32, MXFP4E1M2_B32) else D


def scales_per_row(qmode: int, D: int) -> int:
    return D // 32 if qmode in BLOCK_MODES else 1


def scale_dtype(qmode: int):
    return np.uint8 if qmode in E8M0_MODES else np.float32


class HostCache:
    """Host copy of one quantized cache: codes [B,H,S,row_bytes] uint8,
    scales [B,H,S,spr] (float32, or uint8 E8M0 for the MX modes), zps [B,H,S] int8
    (affine modes).  ``fill`` writes the sentinel pattern used to detect
    stray writes and reads: codes 0xA5, scales NaN / 0xFF, zp 0x5A."""

    def __init__(self, qmode, B, H, S, D, fill=True):
        self.qmode, self.B, self.H, self.S, self.D = qmode, B, H, S, D
        self.codes = np.empty((B, H, S, row_bytes(qmode, D)), np.uint8)
        self.scales = np.empty((B, H, S, scales_per_row(qmode, D)), scale_dtype(qmode))
        self.zps = np.empty((B, H, S), np.int8) if qmode in (INT8_TH, UINT4_TH) else None
        if fill:
            self.sentinel_fill()

    def sentinel_fill(self):
        self.codes.fill(0xA5)
        if self.scales.dtype == np.uint8:
            self.scales.fill(0xFF)
        else:
            self.scales.fill(np.nan)
        if self.zps is not None:
            self.zps.fill(0x5A)

    def copy(self):
        c = HostCache(self.qmode, self.B, self.H, self.S, self.D, fill=False)
        c.codes[...] = self.codes
        c.scales[...] = self.scales
        if self.zps is not None:
            c.zps[...] = self.zps
        return c


def quantize_rows(qmode, x, flags=0):
    """Quantize rows x[..., D] (float32) -> (codes, scales, zps).  flags:
    MX_SCALE_OCP for the MX modes."""
    x = _c(np.asarray(x, dtype=np.float32), np.float32)
    D = x.shape[-1]
    n = x.size // D
    codes = np.empty(x.shape[:-1] + (row_bytes(qmode, D),), np.uint8)
    scales = np.empty(x.shape[:-1] + (scales_per_row(qmode, D),), scale_dtype(qmode))
    zps = np.empty(x.shape[:-1], np.int8)
    lib().orc_quantize_rows_f(qmode, int(flags), _ptr(x), n, D, _ptr(codes), _ptr(scales), _ptr(zps))
    return codes, scales, (zps if qmode in (INT8_TH, UINT4_TH) else None)


def dequantize_rows(qmode, codes, scales, zps, D):
    codes = _c(codes, np.uint8)
    scales = _c(scales, scale_dtype(qmode))
    n = codes.size // row_bytes(qmode, D)
    out = np.empty(codes.shape[:-1] + (D,), np.float64)
    z = None if zps is None else _c(zps, np.int8)
    lib().orc_dequantize_rows(qmode, _ptr(codes), _ptr(scales), _ptr(z), n, D, _ptr(out))
    return out


def quant_scatter(cache: HostCache, x, slot_mapping, slot_stride_b=None, parallel=False, qflags=0):
    """Quantize x[B,H,T,D] (float32 values) and scatter into ``cache`` in place.
    slot_mapping is int32 [B,T] (or [T] with slot_stride_b=0); qflags:
    MX_SCALE_OCP for the MX modes.  Returns the error flags."""
    x = _c(np.asarray(x, dtype=np.float32), np.float32)
    B, H, T, D = x.shape
    if (B, H, D) != (cache.B, cache.H, cache.D):
        raise ValueError("x shape does not match the cache")
    sm = _c(np.asarray(slot_mapping, dtype=np.int32), np.int32)
    if slot_stride_b is None:
        slot_stride_b = 0 if sm.ndim == 1 else sm.shape[-1]
    f = lib().orc_quant_scatter_par_f if parallel else lib().orc_quant_scatter_f
    return f(cache.qmode, int(qflags), _ptr(x), B, H, T, D, _ptr(sm), slot_stride_b, cache.S,
             _ptr(cache.codes), _ptr(cache.scales), _ptr(cache.zps))


def positions_sink(start_pos, T, sink, window, cache_positions=None):
    """Slots for positions start_pos..start_pos+T-1 (sink/ring layout).
    Updates cache_positions (int32 [sink+window]) in place if given."""
    sm = np.empty(T, np.int32)
    cp = None if cache_positions is None else cache_positions
    if cp is not None and (cp.dtype != np.int32 or not cp.flags.c_contiguous):
        raise TypeError("cache_positions must be contiguous int32")
    lib().orc_positions_sink(start_pos, T, sink, window, _ptr(sm), _ptr(cp))
    return sm


def positions_full(start_pos, T, capacity, cache_positions=None):
    sm = np.empty(T, np.int32)
    cp = cache_positions
    flags = lib().orc_positions_full(start_pos, T, capacity, _ptr(sm), _ptr(cp))
    return sm, flags


def build_mask(cache_positions, p0, Lq, sink, window):
    cp = _c(cache_positions, np.int32)
    S = cp.shape[0]
    mask = np.empty((Lq, S), np.float32)
    lib().orc_build_mask(_ptr(cp), S, p0, Lq, sink, window, _ptr(mask))
    return mask


def sdpa(q, kc: HostCache, vc: HostCache, kv_len, mask=None, causal=False,
         sm_scale=None, rows=None):
    """Attention on the quantized caches in fp64.

    q: [B,Hq,Lq,D] (any float dtype; widened to fp64 exactly).
    mask: None, [Lq,S] (shared over batch) or [B,Lq,S] float32.
    rows: None for all outputs ([B,Hq,Lq,D]); or int array [n,3] of
    (b, h, r) to compute only those rows ([n,D])."""
    q = np.ascontiguousarray(np.asarray(q, dtype=np.float64))
    B, Hq, Lq, D = q.shape
    if kc.qmode != vc.qmode:
        raise ValueError("K and V caches must share a quantization mode")
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(D)
    m = None
    mstride = 0
    if mask is not None:
        m = _c(mask, np.float32)
        mstride = 0 if m.ndim == 2 else Lq * kc.S
    args = [_ptr(q), B, Hq, Lq, kc.qmode, kc.H, kc.S, D,
            _ptr(kc.codes), _ptr(kc.scales), _ptr(kc.zps),
            _ptr(vc.codes), _ptr(vc.scales), _ptr(vc.zps),
            int(kv_len), _ptr(m), mstride, int(bool(causal)), float(sm_scale)]
    if rows is None:
        out = np.empty((B, Hq, Lq, D), np.float64)
        flags = lib().orc_sdpa(*args, _ptr(out))
    else:
        r = _c(np.asarray(rows, dtype=np.int32).reshape(-1, 3), np.int32)
        out = np.empty((r.shape[0], D), np.float64)
        flags = lib().orc_sdpa_rows(*args, _ptr(r), r.shape[0], _ptr(out))
    if flags:
        raise ValueError(f"oracle rejected kv_len={kv_len} (flags {flags})")
    return out
