// kvq_device.h -- device helpers shared by the gfx950 kernels of libkvq.
// (Product code: nothing here is shared with the CPU oracle.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// bf16 <-> fp32 (bit level; bf16 -> fp32 is exact)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 with round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Load 8 consecutive input elements as fp32 (16-byte aligned for bf16,
// 32-byte span for fp32).
template <bool BF16>
__device__ __forceinline__ void load8(const void* base, int64_t elem_off, float v[8]) {
    if constexpr (BF16) {
        const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + elem_off);
        v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
        v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
        v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
        v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
    } else {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + elem_off);
        const float4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}

// ---------------------------------------------------------------------------
// E8M0 scales and element encoders
// ---------------------------------------------------------------------------

// Biased E8M0 exponent of the smallest power of two >= s (s >= 0), clamped
// to [0, 254].
__device__ __forceinline__ uint32_t e8m0_ceil(float s) {
    if (!(s > 0.0f)) return 0u;
    const uint32_t u = __float_as_uint(s);
    const int ef = (int)(u >> 23);
    const uint32_t mant = u & 0x7FFFFFu;
    int e;
    if (ef == 0) e = (32 - (int)__clz(mant - 1u)) - 149;   // ceil(log2(mant * 2^-149))
    else e = ef - 127 + (mant != 0u ? 1 : 0);
    int b = e + 127;
    b = b < 0 ? 0 : (b > 254 ? 254 : b);
    return (uint32_t)b;
}

// Biased E8M0 exponent floor(log2 amax) - emax + 127 (OCP MX shared-scale
// rule), clamped to [0, 254]; 0 for amax == 0.
__device__ __forceinline__ uint32_t e8m0_floor(float amax, int emax) {
    if (!(amax > 0.0f)) return 0u;
    const uint32_t u = __float_as_uint(amax);
    const int ef = (int)(u >> 23);
    const int fl = ef == 0 ? (31 - (int)__clz(u & 0x7FFFFFu)) - 149 : ef - 127;
    int b = fl - emax + 127;
    b = b < 0 ? 0 : (b > 254 ? 254 : b);
    return (uint32_t)b;
}

__device__ __forceinline__ float e8m0_value(uint32_t b) {
    return b == 0u ? __uint_as_float(0x00400000u) : __uint_as_float(b << 23);
}

// Element encoders: FP8 E4M3FN, FP8 E5M2 and FP4 E2M1 codes, round to nearest
// even, |y| at or above the format's largest value (448, 57344, 6) saturating
// to it, sign kept (a NaN saturates too).  The gfx950 conversion instructions
// round to nearest even; |y| is clamped to the largest value first, which
// gives the saturation and turns a NaN into that value with its sign kept.
// tests/csrc/encoder_sweep.hip compares these with bit-level encoders over
// all 2^32 fp32 inputs.  Codes of y[0..3] go to bytes 0..3 (FP8); E2M1 codes
// of y[0..7] to nibbles 0..7.
__device__ __forceinline__ float clamp_mag(float y, float mx) {
    return __builtin_copysignf(fminf(__builtin_fabsf(y), mx), y);
}
__device__ __forceinline__ uint32_t cvt4_e4m3fn(const float* y) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_mag(y[0], 448.0f), clamp_mag(y[1], 448.0f), 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp_mag(y[2], 448.0f), clamp_mag(y[3], 448.0f), lo, true);
}
__device__ __forceinline__ uint32_t cvt4_e5m2(const float* y) {
    const int lo = __builtin_amdgcn_cvt_pk_bf8_f32(clamp_mag(y[0], 57344.0f), clamp_mag(y[1], 57344.0f), 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(clamp_mag(y[2], 57344.0f), clamp_mag(y[3], 57344.0f), lo, true);
}
// FP4-E1M2 (sign, one exponent bit of bias 0, two mantissa bits): the
// magnitudes k / 2, k = 0..7, are evenly spaced, so the code of y is
// rne(2 |y|) with 2 |y| clamped to 7 (a NaN too), y's sign in bit 3.
__device__ __forceinline__ uint32_t cvt8_e1m2(const float* y) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float k = __builtin_rintf(fminf(2.0f * __builtin_fabsf(y[i]), 7.0f));
        w |= ((uint32_t)k | ((__float_as_uint(y[i]) >> 28) & 8u)) << (4 * i);
    }
    return w;
}
// Elements 2j and 2j + 1 of eight FP4-E1M2 codes (element i in nibble i of
// w) as an exact fp16 pair: in [512, 1024) the fp16 ulp is 1/2, so magnitude
// code k placed in the mantissa of 512 (0x6000) reads 512 + k / 2, and
// subtracting 512 under the same sign leaves +-k / 2.
__device__ __forceinline__ uint32_t e1m2_pair_h2(uint32_t w, int j) {
    const uint32_t n = (w >> (8 * j)) & 0xFFu;                          // the two codes
    const uint32_t sg = ((n & 0x8u) << 12) | ((n & 0x80u) << 24);       // their fp16 sign bits
    const uint32_t a = 0x60006000u | sg | (n & 0x7u) | ((n & 0x70u) << 12);
    const uint32_t b = 0x60006000u | sg;
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, a) - __builtin_bit_cast(half2_t, b));
}
__device__ __forceinline__ uint32_t cvt8_e2m1(const float* y) {
    uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, clamp_mag(y[0], 6.0f), clamp_mag(y[1], 6.0f), 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, clamp_mag(y[2], 6.0f), clamp_mag(y[3], 6.0f), 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, clamp_mag(y[4], 6.0f), clamp_mag(y[5], 6.0f), 1.0f, 2);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, clamp_mag(y[6], 6.0f), clamp_mag(y[7], 6.0f), 1.0f, 3);
}

// ---------------------------------------------------------------------------
// Cross-lane helpers (wave64)
// ---------------------------------------------------------------------------
// v of lane (l ^ 1), (l ^ 2) by quad permutes; once every lane of a quad
// (octet) holds the same value, the half mirror (mirror) of a row of 16
// brings in the other quad's (octet's) value; across the two rows of a
// 32-lane half by a swizzle (xor 16), across the halves by a shuffle.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// max / min over aligned groups of WIDTH lanes; every lane gets its group's
// result (min and max are exact, so the pairing order does not matter)
template <int WIDTH, bool MAX>
__device__ __forceinline__ float wave_reduce_sub(float v) {
    auto op = [](float a, float b) __attribute__((always_inline)) { return MAX ? fmaxf(a, b) : fminf(a, b); };
    if constexpr (WIDTH >= 2) v = op(v, dpp_f<0xB1>(v));     // quad_perm [1, 0, 3, 2]
    if constexpr (WIDTH >= 4) v = op(v, dpp_f<0x4E>(v));     // quad_perm [2, 3, 0, 1]
    if constexpr (WIDTH >= 8) v = op(v, dpp_f<0x141>(v));    // row_half_mirror
    if constexpr (WIDTH >= 16) v = op(v, dpp_f<0x140>(v));   // row_mirror
    if constexpr (WIDTH >= 32) v = op(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F)));
    if constexpr (WIDTH >= 64) v = op(v, __shfl_xor(v, 32, 64));
    return v;
}
template <int WIDTH>
__device__ __forceinline__ float wave_max_sub(float v) { return wave_reduce_sub<WIDTH, true>(v); }
template <int WIDTH>
__device__ __forceinline__ float wave_min_sub(float v) { return wave_reduce_sub<WIDTH, false>(v); }

}  // namespace kvq
