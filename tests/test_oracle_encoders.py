"""Pins for the oracle's element encoders (FP8-E4M3FN, FP4-E2M1, FP4-E1M2, E8M0).

Each encoder is checked against an exhaustive nearest-grid search written from
the format definitions alone (every code enumerated, its value computed from
sign/exponent/mantissa, nearest by absolute distance, ties to the even code),
and FP8 additionally against torch's own float8_e4m3fn cast.  Format and
rounding rules: IndexerQuantCache page, "function description" (per-block
formula; FP8 / MX-FP4 modes) and the parameter table (FP4 packed two per uint8,
E8M0 scales).
"""
import numpy as np
import pytest
import torch


def _e4m3_grid():
    """Finite non-negative E4M3FN values, index = 7-bit magnitude code."""
    vals = []
    for code in range(0x7F):  # 0x7F is NaN
        e, m = code >> 3, code & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals, np.float64)


def _e2m1_grid():
    vals = []
    for code in range(8):
        e, m = code >> 1, code & 1
        vals.append(m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1))
    return np.array(vals, np.float64)


def _e1m2_grid():
    """FP4-E1M2 magnitudes from the bit fields: one exponent bit (bias 0, the
    IEEE rule 2^(k-1) - 1 for k = 1), two mantissa bits; exponent 0 is
    subnormal.  Index = 3-bit magnitude code."""
    vals = []
    for code in range(8):
        e, m = code >> 2, code & 3
        vals.append(m / 4 * 2.0 ** 1 if e == 0 else (1 + m / 4) * 2.0 ** (e - 0))
    return np.array(vals, np.float64)


def _nearest_even(y, grid, sign_bit):
    """Brute force: nearest grid magnitude, ties to the even code; sign kept."""
    # beyond the largest grid value the nearest is that value; clipping keeps
    # the float64 distances exact for the comparison
    a = np.minimum(np.abs(y.astype(np.float64)), 2.0 ** 20)
    dist = np.abs(a[:, None] - grid[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    codes = np.arange(grid.size)
    # among tied candidates prefer the even code (there are at most two)
    even = cand & (codes[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    sign = np.signbit(y).astype(np.uint8) * sign_bit
    return (pick.astype(np.uint8) | sign).astype(np.uint8)


def _all_finite_bf16_as_f32():
    bits = np.arange(65536, dtype=np.uint32) << 16
    y = bits.view(np.float32)
    return y[np.isfinite(y)]


def test_e4m3_grid_is_the_format():
    g = _e4m3_grid()
    assert g[0x7E] == 448.0 and g[1] == 2.0 ** -9 and g[8] == 2.0 ** -6
    assert np.all(np.diff(g) > 0)


def test_e4m3_exhaustive_bf16(orc):
    y = _all_finite_bf16_as_f32()
    got = orc.e4m3fn_encode(y)
    want = _nearest_even(y, _e4m3_grid(), 0x80)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first y={y[bad[:5]]} got={got[bad[:5]]} want={want[bad[:5]]}"


def test_e4m3_midpoints_and_random(orc):
    g = _e4m3_grid()
    mids = ((g[1:] + g[:-1]) / 2).astype(np.float32)   # exact in fp32
    r = np.random.default_rng(7)
    rand = (r.standard_normal(20000) * r.choice([1e-3, 0.1, 1, 30, 300], 20000)).astype(np.float32)
    y = np.concatenate([mids, -mids, np.nextafter(mids, np.float32(0)),
                        np.nextafter(mids, np.float32(1e9)), rand,
                        np.array([448, 449, 463.9, 464, 465, 1e30, -1e30, 0.0, -0.0], np.float32)])
    assert np.array_equal(orc.e4m3fn_encode(y), _nearest_even(y, g, 0x80))


def test_e4m3_against_torch_cast(orc):
    """torch's float8_e4m3fn cast (a library routine), away from saturation."""
    y = _all_finite_bf16_as_f32()
    y = y[np.abs(y) < 448]
    r = np.random.default_rng(3)
    y = np.concatenate([y, (r.standard_normal(50000) * 50).astype(np.float32)])
    y = y[np.abs(y) < 448]
    want = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.e4m3fn_encode(y), want)


def test_e4m3_saturation_and_sign(orc):
    assert orc.e4m3fn_encode([1e6])[0] == 0x7E
    assert orc.e4m3fn_encode([-1e6])[0] == 0xFE
    assert orc.e4m3fn_encode([-0.0])[0] == 0x80           # keeps the sign
    assert orc.e4m3fn_encode([-2.0 ** -11])[0] == 0x80    # rounds to -0
    assert orc.e4m3fn_encode([2.0 ** -10])[0] == 0x00     # tie -> even (0)
    assert orc.e4m3fn_encode([3 * 2.0 ** -10])[0] == 0x02  # tie 1.5 steps -> 2
    for c in range(0x7F):
        assert orc.e4m3fn_encode([orc.e4m3fn_decode(c)])[0] == c


def test_e2m1_exhaustive_bf16(orc):
    y = _all_finite_bf16_as_f32()
    assert np.array_equal(orc.e2m1_encode(y), _nearest_even(y, _e2m1_grid(), 0x8))


def test_e2m1_ties(orc):
    # 0.25 -> 0 (code 0), 0.75 -> 1.0 (code 2), 1.25 -> 1.0 (2), 1.75 -> 2.0 (4),
    # 2.5 -> 2.0 (4), 3.5 -> 4.0 (6), 5 -> 4.0 (6); >= 6 saturates to 7.
    y = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 100.0, -0.1], np.float32)
    assert list(orc.e2m1_encode(y)) == [0, 2, 2, 4, 4, 6, 6, 7, 7, 7, 8]
    for c in range(16):
        v = orc.e2m1_decode(c)
        assert orc.e2m1_encode([v])[0] == c


def test_e1m2_grid_is_the_format(orc):
    # the 8 magnitudes are evenly spaced: the subnormal step equals the normal one
    assert list(_e1m2_grid()) == [0.0, 0.5, 1.0, 1.5, 2.0, 2.5, 3.0, 3.5]
    for c in range(16):
        v = orc.e1m2_decode(c)
        assert v == (-1.0 if c & 8 else 1.0) * _e1m2_grid()[c & 7]
        assert np.signbit(v) == bool(c & 8)


def test_e1m2_exhaustive_bf16(orc):
    y = _all_finite_bf16_as_f32()
    assert np.array_equal(orc.e1m2_encode(y), _nearest_even(y, _e1m2_grid(), 0x8))


def test_e1m2_ties(orc):
    # 0.25 -> 0 (codes 0|1 tie, even 0), 0.75 -> 1.0 (1|2 -> 2), 1.25 -> 1.0 (2|3 -> 2),
    # 1.75 -> 2.0 (3|4 -> 4), 2.25 -> 2.0 (4|5 -> 4), 2.75 -> 3.0 (5|6 -> 6),
    # 3.25 -> 3.0 (6|7 -> 6); >= 3.5 saturates to 7; -0.1 -> -0 (code 8).
    y = np.array([0.25, 0.75, 1.25, 1.75, 2.25, 2.75, 3.25, 3.5, 3.75, 100.0, -0.1], np.float32)
    assert list(orc.e1m2_encode(y)) == [0, 2, 2, 4, 4, 6, 6, 7, 7, 7, 8]
    for c in range(16):
        assert orc.e1m2_encode([orc.e1m2_decode(c)])[0] == c


def test_e8m0_smallest_power_of_two_at_or_above(orc):
    """E8M0 exponent b: X = 2^(b-127) satisfies X >= s > X/2 (reading: the
    MX scale is rounded up so that no element of the block clips)."""
    pos = _all_finite_bf16_as_f32()
    pos = pos[pos > 0]
    r = np.random.default_rng(11)
    rand = np.abs(r.standard_normal(100000)).astype(np.float32) * \
        np.float32(2.0) ** r.integers(-140, 120, 100000).astype(np.float32)
    s = np.concatenate([pos, rand[rand > 0]])
    b = orc.e8m0_ceil(s).astype(np.int64)
    X = np.ldexp(1.0, b - 127)
    inside = (b > 0) & (b < 254)
    assert np.all(X[inside] >= s[inside]) and np.all(X[inside] / 2 < s[inside])
    # clamped ends: tiny s -> 0, huge s -> 254 (0xFF is never produced)
    assert np.all(s[b == 0] <= 2.0 ** -127)
    assert np.all(s[b == 254] > 2.0 ** 126)
    assert orc.e8m0_ceil([0.0])[0] == 0
    assert list(orc.e8m0_ceil([1.0, 1.5, 2.0, 0.75, 2.0 ** -127, 2.0 ** -126 * 1.5])) == \
        [127, 128, 128, 127, 0, 2]


def _e5m2_grid():
    """Finite non-negative E5M2 values, index = 7-bit magnitude code (bias 15,
    2 mantissa bits; exponent 31 is inf / NaN)."""
    vals = []
    for code in range(0x7C):
        e, m = code >> 2, code & 3
        vals.append(m * 2.0 ** -16 if e == 0 else (1 + m / 4) * 2.0 ** (e - 15))
    return np.array(vals, np.float64)


def test_e5m2_grid_is_the_format():
    g = _e5m2_grid()
    assert g[0x7B] == 57344.0 and g[1] == 2.0 ** -16 and g[4] == 2.0 ** -14
    assert np.all(np.diff(g) > 0)


def test_e5m2_decode_is_the_top_byte_of_fp16(orc):
    """E5M2 is fp16 with the low mantissa byte dropped: code c decodes to the
    fp16 value with bits c << 8 (inf and NaN codes included)."""
    for c in range(256):
        h = np.array([c << 8], np.uint16).view(np.float16)[0]
        v = orc.e5m2_decode(c)
        assert (np.isnan(h) and np.isnan(v)) or (float(h) == v and np.signbit(h) == np.signbit(v)), c


def test_e5m2_exhaustive_bf16(orc):
    y = _all_finite_bf16_as_f32()
    got = orc.e5m2_encode(y)
    want = _nearest_even(y, _e5m2_grid(), 0x80)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first y={y[bad[:5]]} got={got[bad[:5]]} want={want[bad[:5]]}"


def test_e5m2_midpoints_and_torch_cast(orc):
    g = _e5m2_grid()
    mids = ((g[1:] + g[:-1]) / 2).astype(np.float32)
    r = np.random.default_rng(17)
    rand = (r.standard_normal(20000) * r.choice([1e-4, 0.1, 1, 300, 20000], 20000)).astype(np.float32)
    y = np.concatenate([mids, -mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)), rand,
                        np.array([57344, 57345, 61439, 61440, 1e30, -1e30, 0.0, -0.0], np.float32)])
    assert np.array_equal(orc.e5m2_encode(y), _nearest_even(y, g, 0x80))
    # torch's float8_e5m2 cast (a library routine), away from saturation
    inside = y[np.abs(y) < 57344]
    want = torch.from_numpy(inside).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(orc.e5m2_encode(inside), want)
    assert orc.e5m2_encode([-0.0])[0] == 0x80 and orc.e5m2_encode([1e9])[0] == 0x7B
    for c in range(0x7C):
        assert orc.e5m2_encode([orc.e5m2_decode(c)])[0] == c


@pytest.mark.parametrize("emax", [2, 8])
def test_e8m0_floor_rule(orc, emax):
    """OCP floor rule: X = 2^(b - 127) with X * 2^emax <= amax < X * 2^(emax+1)
    inside the E8M0 range; amax = 0 gives 0; the ends clamp to [0, 254]."""
    pos = _all_finite_bf16_as_f32()
    pos = pos[pos > 0]
    r = np.random.default_rng(13)
    rand = np.abs(r.standard_normal(100000)).astype(np.float32) * \
        np.float32(2.0) ** r.integers(-140, 120, 100000).astype(np.float32)
    a = np.concatenate([pos, rand[rand > 0]])
    b = orc.e8m0_floor(a, emax).astype(np.int64)
    X = np.ldexp(1.0, b - 127)
    inside = (b > 0) & (b < 254)
    ratio = a[inside].astype(np.float64) / X[inside]
    assert np.all(ratio >= 2.0 ** emax) and np.all(ratio < 2.0 ** (emax + 1))
    assert orc.e8m0_floor([0.0], emax)[0] == 0
    assert orc.e8m0_floor([3e38], emax)[0] == 127 + 127 - emax
    assert orc.e8m0_floor([1e-44], emax)[0] == 0
