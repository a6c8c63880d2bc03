"""Seeded synthetic inputs for the five workloads.

This module holds only random-number generation and shapes: none of the
method's arithmetic.  The oracle and the HIP path both draw their inputs from
here, so identical bytes reach both sides.

Every stream comes from ``numpy.random.default_rng(SeedSequence([1000 + cfg,
stream, block]))`` with stream 0 = Q, 1 = K, 2 = V, 3 = slots, 4 = outlier
channels, 5 = outlier mask, and ``block`` the decode step or 2048-position
block.  Values are float32 N(0, 1); where a workload is bf16 they are rounded
to bf16 (round to nearest even, by torch's dtype cast) and widened back, so the
float32 array holds exactly the bf16 values.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

Q, K, V, SLOTS, OUTLIER_CH, OUTLIER_MASK = 0, 1, 2, 3, 4, 5


def rng(cfg: int, stream: int, block: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([1000 + cfg, stream, block]))


def normal(cfg: int, stream: int, block: int, shape, bf16: bool) -> np.ndarray:
    """float32 N(0,1) of ``shape``; rounded to bf16 values if ``bf16``."""
    x = rng(cfg, stream, block).standard_normal(size=shape, dtype=np.float32)
    if bf16:
        x = to_bf16_values(x)
    return x


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """float32 array holding the bf16 (RNE) rounding of ``x``."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).float().numpy()


def as_torch(x: np.ndarray, bf16: bool) -> torch.Tensor:
    """CPU tensor in the workload's input dtype (exact: x holds bf16 values)."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(torch.bfloat16) if bf16 else t


# --------------------------------------------------------------------------
# Workload shapes
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Tiny:
    """Tiny full-context int8 cache: B1, 4 q heads over 2 KV heads, D64,
    256 slots; fp32 Q/K/V; prefill 64 tokens then 32 decode steps."""
    cfg: int = 1
    B: int = 1
    Hq: int = 4
    Hkv: int = 2
    D: int = 64
    S: int = 256
    prefill: int = 64
    decode_steps: int = 32
    bf16: bool = False


@dataclass(frozen=True)
class Llama8BDecode:
    """Llama-3-8B-shaped decode layer: B8, 32/8 heads, D128, 8192 slots,
    kv_len 4096 (history 0..4094, new token at 4095); bf16; 4 of every 128
    channels of K and of V scaled x10 (seeded per KV head, fixed over
    tokens; K and V draw separate sets)."""
    cfg: int = 2
    B: int = 8
    Hq: int = 32
    Hkv: int = 8
    D: int = 128
    S: int = 8192
    kv_len: int = 4096
    n_outlier: int = 4
    outlier_gain: float = 10.0
    bf16: bool = True


@dataclass(frozen=True)
class SinkRing:
    """Attention-sink (2048 slots = 4 sink + 2044 window) and ring (1024)
    caches; B4, 32/8 heads, D128, bf16 N(0,1); decode positions 0..6000."""
    cfg: int = 3
    B: int = 4
    Hq: int = 32
    Hkv: int = 8
    D: int = 128
    sink: int = 4
    window: int = 2044
    ring_window: int = 1024
    last_pos: int = 6000
    bf16: bool = True


@dataclass(frozen=True)
class LongPrefill:
    """Long-context chunked prefill: B1, 32/16 heads, D256, 131072 slots,
    4-bit cache; bf16 chunks of 2048 ending (exclusive) at 65536 and 131072."""
    cfg: int = 4
    B: int = 1
    Hq: int = 32
    Hkv: int = 16
    D: int = 256
    S: int = 131072
    Lq: int = 2048
    chunk_ends: tuple = (65536, 131072)
    bf16: bool = True


@dataclass(frozen=True)
class BlockScatter:
    """Block-quantized scatter: x [16384, 128] bf16 N(0,1), 1% of entries
    x20; 16384 distinct slots out of 65536, 1638 of them set to -1."""
    cfg: int = 5
    bs: int = 16384
    d: int = 128
    n_slots: int = 65536
    outlier_frac: float = 0.01
    outlier_gain: float = 20.0
    n_skip: int = 1638
    bf16: bool = True


TINY, LLAMA8B, SINKRING, LONGPREFILL, BLOCKSCATTER = (
    Tiny(), Llama8BDecode(), SinkRing(), LongPrefill(), BlockScatter())


# --------------------------------------------------------------------------
# Generators
# --------------------------------------------------------------------------

def tiny_prefill(w: Tiny = TINY):
    """(q, k, v) for the 64-token prefill: q [B,Hq,T,D], k/v [B,Hkv,T,D]."""
    T = w.prefill
    q = normal(w.cfg, Q, 0, (w.B, w.Hq, T, w.D), w.bf16)
    k = normal(w.cfg, K, 0, (w.B, w.Hkv, T, w.D), w.bf16)
    v = normal(w.cfg, V, 0, (w.B, w.Hkv, T, w.D), w.bf16)
    return q, k, v


def tiny_decode(p: int, w: Tiny = TINY):
    """(q, k, v) for the decode step at position p (T = 1)."""
    q = normal(w.cfg, Q, p, (w.B, w.Hq, 1, w.D), w.bf16)
    k = normal(w.cfg, K, p, (w.B, w.Hkv, 1, w.D), w.bf16)
    v = normal(w.cfg, V, p, (w.B, w.Hkv, 1, w.D), w.bf16)
    return q, k, v


def _outlier_channels(w: Llama8BDecode, which: int) -> np.ndarray:
    """[Hkv, n_outlier] channel indices for K (which=1) or V (which=2)."""
    g = rng(w.cfg, OUTLIER_CH, which)
    return np.stack([g.choice(w.D, size=w.n_outlier, replace=False) for _ in range(w.Hkv)])


def llama8b_kv(w: Llama8BDecode = LLAMA8B, batches=None):
    """K and V for positions 0..kv_len-1: [B, Hkv, kv_len, D] each (bf16
    values, outlier channels applied before rounding).  ``batches`` selects
    a subset of batch rows (same values as in the full draw)."""
    out = []
    for which in (K, V):
        x = rng(w.cfg, which, 0).standard_normal(size=(w.B, w.Hkv, w.kv_len, w.D),
                                                 dtype=np.float32)
        ch = _outlier_channels(w, which)
        for h in range(w.Hkv):
            x[:, h, :, ch[h]] *= np.float32(w.outlier_gain)
        if batches is not None:
            x = x[batches]
        out.append(to_bf16_values(x) if w.bf16 else x)
    return out[0], out[1]


def llama8b_q(w: Llama8BDecode = LLAMA8B):
    return normal(w.cfg, Q, 0, (w.B, w.Hq, 1, w.D), w.bf16)


def sinkring_step(p: int, w: SinkRing = SINKRING):
    """(q [B,Hq,1,D], k [B,Hkv,1,D], v [B,Hkv,1,D]) for decode position p."""
    q = normal(w.cfg, Q, p, (w.B, w.Hq, 1, w.D), w.bf16)
    k = normal(w.cfg, K, p, (w.B, w.Hkv, 1, w.D), w.bf16)
    v = normal(w.cfg, V, p, (w.B, w.Hkv, 1, w.D), w.bf16)
    return q, k, v


def longprefill_block(block: int, w: LongPrefill = LONGPREFILL, heads=None):
    """K and V for positions [2048*block, 2048*(block+1)): [B, Hkv, 2048, D]
    (``heads`` selects KV heads, same values as in the full draw)."""
    out = []
    for which in (K, V):
        x = normal(w.cfg, which, block, (w.B, w.Hkv, w.Lq, w.D), False)
        if heads is not None:
            x = x[:, heads]
        out.append(to_bf16_values(x) if w.bf16 else x)
    return out[0], out[1]


def longprefill_q(chunk_end: int, w: LongPrefill = LONGPREFILL):
    """Q of the chunk ending (exclusive) at chunk_end: [B, Hq, 2048, D]."""
    return normal(w.cfg, Q, chunk_end // w.Lq - 1, (w.B, w.Hq, w.Lq, w.D), w.bf16)


def blockscatter_inputs(w: BlockScatter = BLOCKSCATTER):
    """(x [bs, d] bf16 values, slot_mapping int32 [bs])."""
    x = rng(w.cfg, K, 0).standard_normal(size=(w.bs, w.d), dtype=np.float32)
    hit = rng(w.cfg, OUTLIER_MASK, 0).random(size=(w.bs, w.d)) < w.outlier_frac
    x[hit] *= np.float32(w.outlier_gain)
    g = rng(w.cfg, SLOTS, 0)
    slots = g.choice(w.n_slots, size=w.bs, replace=False).astype(np.int32)
    skip = g.choice(w.bs, size=w.n_skip, replace=False)
    slots[skip] = -1
    return (to_bf16_values(x) if w.bf16 else x), slots
