// sdpa_decode.hip -- split-K decode attention (Lq = 1) over a quantized cache.
//
// What is computed: abaddon attention_cache, KvCache::forward_attention (q
// [batch, heads, q_len, head_dim], GQA expansion by repeat_kv, softmax scale);
// the KV loop stops at the filled length kv_len, a device int32 scalar
// (pytorch/executorch PR 20351, kv_len note); ring and sink caches add a 0 /
// -inf float mask (PR 24473, Summary).  Dequantization (code - zp) * scale
// happens in registers and is never materialized.
//
// Mapping on gfx950:
//  * grid (splits, Hkv, B); a 256-thread workgroup (4 waves) owns one
//    (b, kv head g) and one contiguous slice of [0, kv_len), derived on the
//    device from kv_len, so the launch shape is fixed across steps.  The split
//    count keeps every workgroup resident in one round (the VGPR and LDS use
//    of the instantiation decides how many fit per CU).
//  * The G = Hq/Hkv query heads of a KV head are processed together: every
//    K/V byte is read from HBM once for all of them.
//  * Per-row metadata of the slice (scales, zero points, mask) is loaded once,
//    cooperatively, into LDS.
//  * Pass 1 (q . k): a K row is split over CK lanes of KB bytes each; codes
//    become exact fp16 integers (code - zp) (a byte permute under the fp16
//    exponent of 1024, then one packed fp16 subtraction) and meet q in
//    v_dot2_f32_f16 with fp32 accumulation.  q is rescaled by one power of
//    two for the G heads so that max|q| lies in [2^-8, 2^15); a bf16 element
//    is then exact in fp16 when it is at least 2^-17 after the rescale (at
//    worst 2^-9 of max|q|); a smaller one rounds on fp16's subnormal grid,
//    an error below 2^-25, i.e. 2^-17 of max|q|.  fp32 q uses a hi + lo pair
//    of fp16 limbs.
//    Row dots go to LDS.  The codes stream through a register ring of PD
//    steps that is refilled right after each slot is converted.
//  * Middle pass (per head, from LDS): score = dot * scale_k * sm_scale *
//    log2(e) + mask, the slice maximum m, p = 2^(score - m), l = sum p, and
//    p * scale_v back to LDS; the zero points enter through one correction
//    sum per head, sum p * scale_v * (zp + offset).
//  * Pass 2 (p . v): a V row is split over CV lanes of 16 bytes; fp32 FMA of
//    p * scale_v on v_cvt_f32_ubyte of the codes; the first PDV steps of the
//    V ring are issued before the middle pass so the V stream overlaps it.
//  * Block caches (per 32 elements: FP8-E4M3 or FP8-E5M2 or int8 with an fp32
//    scale, MX-FP8 / MX-FP4 with an E8M0 scale; the IndexerQuantCache operator
//    page's per-block formats): codes become exact fp16 / fp32 values (the
//    gfx950 conversion instructions, or the exponent trick for int8); a 16-byte chunk of a lane lies inside one
//    block, so the block scale travels in the load ring with the codes and
//    multiplies the chunk's partial q . k (pass 1) or p (pass 2).  Rows carry
//    no scale or zero point of their own.
//  * Merge: a reduce-scatter of the accumulators across the row groups of a
//    wave (lane-swap permutes and DPP), then the waves through LDS; one
//    partial (m, l, o[D]) per (b, head, split) goes to the workspace.  A small
//    combine kernel merges the splits (a separate launch: merging inside the
//    split kernel would need a device-scope release/acquire per workgroup,
//    which on this multi-XCD part writes back and invalidates L2).
//  * Loads use global (not flat) addressing so that waits for LDS never wait
//    for loads in flight, and the ring loops have no data-dependent branches:
//    steps past a wave's rows run on a clamped row and store nothing.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

struct DecodeArgs {
    const void* q;
    int B, Hq, Hkv, S;
    const uint8_t* kc;
    const float* ks;
    const int8_t* kz;
    const uint8_t* vc;
    const float* vs;
    const int8_t* vz;
    const int32_t* kv_len;
    int kv_len_sb;         // 0: one kv_len for the batch; 1: one per batch row
    const float* mask;
    int64_t mask_sb;
    float sm_scale_log2;   // sm_scale * log2(e)
    float* part_o;         // [B, Hq, splits, D]
    float* part_ml;        // [B, Hq, splits, 2]
    int32_t* err;
};

constexpr int DEC_WAVES = 4;
constexpr int DEC_CHUNK_ALIGN = 32;   // split slices start on multiples of 32 rows

__device__ __forceinline__ half2_t as_h2(uint32_t w) { return __builtin_bit_cast(half2_t, w); }

__device__ __forceinline__ uint32_t h2_sub(uint32_t a, uint32_t b) {
    half2_t r = __builtin_bit_cast(half2_t, a) - __builtin_bit_cast(half2_t, b);
    return __builtin_bit_cast(uint32_t, r);
}

// Exact fp16 values (code - zp) of 16 code bytes (int8: 16 codes, 4-bit: 32)
// as pairs of consecutive elements.  Bytes are placed under the fp16 exponent
// of 1024 by a byte permute (1024 + u, u = code ^ 0x80 for int8, u = code for
// 4-bit) and zoff = (1024 + 128 + zp) resp. (1024 + zp) is subtracted: the
// difference is a small integer, so the subtraction is exact.
template <bool U4>
__device__ __forceinline__ void codes_to_h2(const uint4 w, uint32_t zoff, uint32_t out[U4 ? 16 : 8]) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    if constexpr (!U4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t u = ws[i] ^ 0x80808080u;                  // c + 128 as unsigned
            out[2 * i] = h2_sub(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u), zoff);      // bytes 0,1
            out[2 * i + 1] = h2_sub(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u), zoff);  // bytes 2,3
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = ws[i] & 0x0F0F0F0Fu;                 // elements 0,2,4,6
            const uint32_t hi = (ws[i] >> 4) & 0x0F0F0F0Fu;          // elements 1,3,5,7
            // pair (2j, 2j+1) = (lo.byte j, hi.byte j) under 0x64 high bytes
            out[4 * i + 0] = h2_sub(__builtin_amdgcn_perm(hi, lo, 0x0C040C00u) | 0x64006400u, zoff);
            out[4 * i + 1] = h2_sub(__builtin_amdgcn_perm(hi, lo, 0x0C050C01u) | 0x64006400u, zoff);
            out[4 * i + 2] = h2_sub(__builtin_amdgcn_perm(hi, lo, 0x0C060C02u) | 0x64006400u, zoff);
            out[4 * i + 3] = h2_sub(__builtin_amdgcn_perm(hi, lo, 0x0C070C03u) | 0x64006400u, zoff);
        }
    }
}

__device__ __forceinline__ uint32_t zoff_pair(int zp, bool u4) {
    const _Float16 h = (_Float16)(float)((u4 ? 1024 : 1152) + zp);
    half2_t v = {h, h};
    return __builtin_bit_cast(uint32_t, v);
}

// fp32 values (u = code + 128 for int8, code for 4-bit) of 16 code bytes.
template <bool U4>
__device__ __forceinline__ void codes_to_f32(const uint4 w, float out[U4 ? 32 : 16]) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    if constexpr (!U4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t u = ws[i] ^ 0x80808080u;
            out[4 * i + 0] = (float)(u & 0xFFu);
            out[4 * i + 1] = (float)((u >> 8) & 0xFFu);
            out[4 * i + 2] = (float)((u >> 16) & 0xFFu);
            out[4 * i + 3] = (float)(u >> 24);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = ws[i] & 0x0F0F0F0Fu;
            const uint32_t hi = (ws[i] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                out[8 * i + 2 * j] = (float)((lo >> (8 * j)) & 0xFFu);
                out[8 * i + 2 * j + 1] = (float)((hi >> (8 * j)) & 0xFFu);
            }
        }
    }
}

// Block-quantized codes to exact fp16 pairs / fp32 values in element order:
// FP8-E4M3FN (MX-FP8 too) and FP8-E5M2 through the gfx950 conversion
// instructions at scale 1 (every E4M3 and E5M2 value is an fp16 value),
// FP4-E2M1 two per byte (element 2i in the low nibble of byte i) the same way,
// int8 as (code + 128) placed under the fp16 exponent of 1024 minus 1152.  The
// per-block scale is applied afterwards, in fp32.
template <int QM>
constexpr bool fp4_mode = QM == QM_MXFP4_B32 || QM == QM_MXFP4E1M2_B32;

template <int QM>
__device__ __forceinline__ void blk_to_h2(const uint4 w, uint32_t out[fp4_mode<QM> ? 16 : 8]) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (QM == QM_MXFP4E1M2_B32) {
#pragma unroll
            for (int j = 0; j < 4; ++j) out[4 * i + j] = e1m2_pair_h2(ws[i], j);
        } else if constexpr (QM == QM_MXFP4_B32) {
            out[4 * i + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ws[i], 1.0f, 0));
            out[4 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ws[i], 1.0f, 1));
            out[4 * i + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ws[i], 1.0f, 2));
            out[4 * i + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ws[i], 1.0f, 3));
        } else if constexpr (QM == QM_FP8E5M2_B32) {
            out[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(ws[i], 1.0f, false));
            out[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(ws[i], 1.0f, true));
        } else if constexpr (QM == QM_INT8_B32) {
            const uint32_t u = ws[i] ^ 0x80808080u;
            out[2 * i] = h2_sub(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u), 0x64806480u);
            out[2 * i + 1] = h2_sub(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u), 0x64806480u);
        } else {
            out[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ws[i], 1.0f, false));
            out[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ws[i], 1.0f, true));
        }
    }
}

template <int QM>
__device__ __forceinline__ void blk_to_f32(const uint4 w, float out[fp4_mode<QM> ? 32 : 16]) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (QM == QM_MXFP4E1M2_B32) {
            // k / 2 with the code's sign (element e in nibble e)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t n = (ws[i] >> (4 * e)) & 0xFu;
                out[8 * i + e] = __uint_as_float(__float_as_uint((float)(n & 7u) * 0.5f) | ((n & 8u) << 28));
            }
        } else if constexpr (QM == QM_MXFP4_B32) {
            const auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ws[i], 1.0f, 0);
            const auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ws[i], 1.0f, 1);
            const auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ws[i], 1.0f, 2);
            const auto v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ws[i], 1.0f, 3);
            out[8 * i + 0] = v0[0]; out[8 * i + 1] = v0[1]; out[8 * i + 2] = v1[0]; out[8 * i + 3] = v1[1];
            out[8 * i + 4] = v2[0]; out[8 * i + 5] = v2[1]; out[8 * i + 6] = v3[0]; out[8 * i + 7] = v3[1];
        } else if constexpr (QM == QM_INT8_B32) {
            const uint32_t u = ws[i] ^ 0x80808080u;          // code + 128
            out[4 * i] = (float)(u & 0xFFu) - 128.0f;
            out[4 * i + 1] = (float)((u >> 8) & 0xFFu) - 128.0f;
            out[4 * i + 2] = (float)((u >> 16) & 0xFFu) - 128.0f;
            out[4 * i + 3] = (float)(u >> 24) - 128.0f;
        } else {
            const auto lo = QM == QM_FP8E5M2_B32 ? __builtin_amdgcn_cvt_pk_f32_bf8(ws[i], false)
                                                 : __builtin_amdgcn_cvt_pk_f32_fp8(ws[i], false);
            const auto hi = QM == QM_FP8E5M2_B32 ? __builtin_amdgcn_cvt_pk_f32_bf8(ws[i], true)
                                                 : __builtin_amdgcn_cvt_pk_f32_fp8(ws[i], true);
            out[4 * i] = lo[0]; out[4 * i + 1] = lo[1]; out[4 * i + 2] = hi[0]; out[4 * i + 3] = hi[1];
        }
    }
}

// A block scale as loaded (fp32 bits, or an E8M0 byte) to its fp32 value;
// E8M0 b is 2^(b - 127), b = 0 being the subnormal 2^-127.
template <bool E8M0>
__device__ __forceinline__ float blk_scale(uint32_t raw) {
    if constexpr (E8M0) return __uint_as_float(raw ? raw << 23 : 0x00400000u);
    else return __uint_as_float(raw);
}

// Cross-lane helpers.  DPP controls: quad_perm [1,0,3,2] (xor 1), quad_perm
// [2,3,0,1] (xor 2), row_half_mirror (lane i <-> 7 - i within 8), row_mirror
// (i <-> 15 - i within 16), row_ror:8 (xor 8 within 16).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140, DPP_ROR8 = 0x128;

// Sum over aligned groups of N lanes (N = 2, 4, 8, 16); every lane gets the sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (N >= 2) v += dpp<DPP_XOR1>(v);
    if constexpr (N >= 4) v += dpp<DPP_XOR2>(v);
    if constexpr (N >= 8) v += dpp<DPP_HALF_MIRROR>(v);
    if constexpr (N >= 16) v += dpp<DPP_MIRROR>(v);
    return v;
}

// Max / sum over all 64 lanes (every lane gets the result).
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<DPP_XOR1>(v));
    v = fmaxf(v, dpp<DPP_XOR2>(v));
    v = fmaxf(v, dpp<DPP_HALF_MIRROR>(v));
    v = fmaxf(v, dpp<DPP_ROR8>(v));
    auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<DPP_XOR1>(v);
    v += dpp<DPP_XOR2>(v);
    v += dpp<DPP_HALF_MIRROR>(v);
    v += dpp<DPP_ROR8>(v);
    auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// One reduce-scatter level across lanes that differ in lane bit O (O = 32,
// 16, 8, 4, 2): pairs (x, y) of the current value list; lanes with the bit
// clear keep x + partner.x, lanes with it set keep y + partner.y.
template <int O>
__device__ __forceinline__ float rs_pair(float x, float y, int lane) {
    if constexpr (O == 32) {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else if constexpr (O == 16) {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else if constexpr (O == 8) {
        const float sx = x + dpp<DPP_ROR8>(x), sy = y + dpp<DPP_ROR8>(y);
        return (lane & 8) ? sy : sx;
    } else {
        const float sx = x + __shfl_xor(x, O, 64), sy = y + __shfl_xor(y, O, 64);
        return (lane & O) ? sy : sx;
    }
}

// Reduce-scatter of N values per lane over the lanes that differ in bits
// [LO, 64): afterwards lane l holds values [blk * N / K, (blk + 1) * N / K)
// summed, K = 64 / LO groups, blk = l / LO.  The result overwrites v[0..N/K).
template <int N, int O, int LO>
__device__ __forceinline__ void reduce_scatter(float* v, int lane) {
    if constexpr (O >= LO) {
#pragma unroll
        for (int i = 0; i < N / 2; ++i) v[i] = rs_pair<O>(v[i], v[i + N / 2], lane);
        reduce_scatter<N / 2, O / 2, LO>(v, lane);
    }
}

// Geometry of the split kernel, shared by the kernel and the host's choice of
// the split count.  K pass: KB code bytes per lane (32 when the fp16 q pairs
// for them fit 64 registers, else 16), CK lanes per row, RK rows per wave
// step; V pass: 16 code bytes per lane, CV lanes per row, RV rows per step.
// A split holds at most rows_max rows (scores in LDS); rows_max is a multiple
// of both workgroup steps.
struct DecGeom {
    int rowb, kb, ck, rk, cv, rv, stepk, stepv, rows_max;
};
__host__ __device__ constexpr DecGeom dec_geom(int D, bool u4, int G) {
    const int rowb = u4 ? D / 2 : D;
    const int kb = (G * 32 * (u4 ? 2 : 1) <= 128 && rowb >= 64) ? 32 : 16;
    const int ck = rowb / kb, rk = 64 / ck;
    const int cv = rowb / 16, rv = 64 / cv;
    const int stepk = rk * DEC_WAVES, stepv = rv * DEC_WAVES;
    const int rows_max = G <= 4 ? 1024 : 512;
    return DecGeom{rowb, kb, ck, rk, cv, rv, stepk, stepv, rows_max};
}

// Sum over aligned groups of N lanes (N = 2, 4, 8, 16) valid in the first
// lane of each group (every level folds into one v_add_f32_dpp).  After the
// two quad levels, row_half_mirror makes lane 0 of an 8-group read lane 7,
// which holds the quad sum of lanes 4..7; row_ror:8 (a rotation by half a
// row, the same in either direction) then adds the other 8-group.
template <int N>
__device__ __forceinline__ float group_sum_first(float v) {
    if constexpr (N >= 2) v += dpp<DPP_XOR1>(v);
    if constexpr (N >= 4) v += dpp<DPP_XOR2>(v);
    if constexpr (N >= 8) v += dpp<DPP_HALF_MIRROR>(v);
    if constexpr (N >= 16) v += dpp<DPP_ROR8>(v);
    return v;
}

// Pointers into global memory.  Keeping the address space explicit makes the
// compiler emit global_load (counted by vmcnt only) instead of flat_load, which
// also counts against lgkmcnt: with flat loads in flight every wait for an LDS
// access would drain the whole prefetch queue.
template <typename T>
using gptr = const __attribute__((address_space(1))) T*;

// Wave-uniform global base pointer (held in SGPRs).
template <typename T>
__device__ __forceinline__ gptr<T> uniform_ptr(const T* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (gptr<T>)(((uint64_t)hi << 32) | lo);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16(gptr<uint8_t> base, uint32_t off) {
    const u32x4_t v = *(gptr<u32x4_t>)(base + off);
    return make_uint4(v.x, v.y, v.z, v.w);
}

#ifndef KVQ_DEC_PD
#define KVQ_DEC_PD 3
#endif
#ifndef KVQ_DEC_PDV
#define KVQ_DEC_PDV 4
#endif

template <int D, int QM, int G, bool QBF16>
__global__ __launch_bounds__(256) void sdpa_decode_split(DecodeArgs a) {
    constexpr bool BLK = QM >= QM_FP8E4M3_B32;      // per-32 block scales, no zero point
    constexpr bool U4 = QM == QM_UINT4_TH || fp4_mode<QM>;             // two codes per byte
    constexpr bool SC8 = fp4_mode<QM> || QM == QM_MXFP8_B32;           // E8M0 block scales
    constexpr int SPR = D / 32;                      // block scales per row
    constexpr int SCB = SC8 ? 1 : 4;                 // bytes per block scale
    constexpr DecGeom GM = dec_geom(D, U4, G);
    constexpr int ROWB = GM.rowb;
    constexpr int EPB = U4 ? 2 : 1;                  // elements per code byte
    constexpr int KB = GM.kb, CK = GM.ck, RK = GM.rk;
    constexpr int NPK = KB * EPB / 2;                // fp16 pairs per lane, K pass
    constexpr int CV = GM.cv, RV = GM.rv;
    constexpr int EV = 16 * EPB;                     // elements per lane, V pass
    constexpr int NL = QBF16 ? 1 : 2;                // fp16 limbs of q
    constexpr float VOFF = (U4 || BLK) ? 0.0f : 128.0f;   // fp32 value = code + VOFF
    constexpr int NV = G * EV;                       // accumulators per lane
    constexpr int NVR = NV / RV;                     // after the row-group reduce-scatter
    constexpr int STEPK = GM.stepk, STEPV = GM.stepv;
    constexpr int PD = KVQ_DEC_PD;                   // K ring depth (steps in flight)
    constexpr int PDV = KVQ_DEC_PDV;                 // V ring depth: issued before the middle pass
    constexpr int ROWS_MAX = GM.rows_max;
    constexpr float NEG_INF = -__builtin_huge_valf();
    constexpr float LOG2E = 1.4426950408889634f;
    static_assert(CK >= 1 && CK <= 16 && CV >= 2 && CV <= 16, "row split");
    static_assert(ROWS_MAX % DEC_CHUNK_ALIGN == 0 && ROWS_MAX <= 4 * 256, "rows_max: 4 metadata rows per thread");

    __shared__ float s_row[ROWS_MAX * G];           // q.k dots, scores, then p * scale_v
    __shared__ float4 s_meta[ROWS_MAX];             // (scale_k, mask, scale_v, zp_v + VOFF)
    __shared__ uint32_t s_kzo[ROWS_MAX];            // fp16 pair of the key zero-point offset
    __shared__ uint32_t s_q[G][NL][D / 2];          // q in fp16 pairs
    __shared__ float s_red[DEC_WAVES][G];
    __shared__ float s_mx[G], s_l[G], s_corr[G];
    __shared__ float s_o[DEC_WAVES][G][D];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int split = blockIdx.x;
    const int nsplit = gridDim.x;
    const int g = blockIdx.y;
    const int b = blockIdx.z;

    // ---- q loads go out first ---------------------------------------------
    constexpr int NQ = G * D;                        // q elements of the group
    constexpr int QPT = ((NQ + 511) / 512) * 2;      // per thread, even
    float qv[QPT];
    {
        const int64_t qoff = ((int64_t)b * a.Hq + g * G) * D;
#pragma unroll
        for (int u = 0; u < QPT; ++u) {
            const int e = min(tid * QPT + u, NQ - 1);
            if constexpr (QBF16) qv[u] = bf16_lo(reinterpret_cast<const uint16_t*>(a.q)[qoff + e]);
            else qv[u] = reinterpret_cast<const float*>(a.q)[qoff + e];
            qv[u] = tid * QPT + u < NQ ? qv[u] : 0.0f;
        }
    }

    // ---- kv_len and this workgroup's slice --------------------------------
    int kv_len = a.kv_len ? a.kv_len[(int64_t)b * a.kv_len_sb] : a.S;
    if (kv_len < 1 || kv_len > a.S) {
        if (a.err && split == 0 && g == 0 && tid == 0) atomicOr(a.err, KVQ_DEV_FLAG_KVLEN);
        kv_len = kv_len < 1 ? 1 : a.S;
    }
    int chunk = (kv_len + nsplit - 1) / nsplit;
    chunk = (chunk + DEC_CHUNK_ALIGN - 1) / DEC_CHUNK_ALIGN * DEC_CHUNK_ALIGN;   // <= ROWS_MAX (host)
    const int j0 = split * chunk;
    const int j1 = min(j0 + chunk, kv_len);          // j1 - 1 is a valid row even when empty
    const int n = max(j1 - j0, 0);
    const int i_last = max(n - 1, 0);                // slice-relative clamp for LDS rows

    const int64_t plane = ((int64_t)b * a.Hkv + g) * a.S;
    const gptr<uint8_t> kbase = uniform_ptr(a.kc + plane * ROWB);
    const gptr<uint8_t> vbase = uniform_ptr(a.vc + plane * ROWB);
    const gptr<float> ksb = uniform_ptr(a.ks + plane);
    const gptr<float> vsb = uniform_ptr(a.vs + plane);
    const gptr<int8_t> kzb = uniform_ptr(a.kz + plane);
    const gptr<int8_t> vzb = uniform_ptr(a.vz + plane);
    // block caches: scale planes [B, Hkv, S, D / 32] of fp32 (FP8) or E8M0 bytes
    const gptr<uint8_t> kscb = uniform_ptr(reinterpret_cast<const uint8_t*>(a.ks) + plane * SPR * SCB);
    const gptr<uint8_t> vscb = uniform_ptr(reinterpret_cast<const uint8_t*>(a.vs) + plane * SPR * SCB);
    const bool has_mask = a.mask != nullptr;
    const gptr<float> mrow = has_mask ? uniform_ptr(a.mask + (int64_t)b * a.mask_sb) : ksb;

    // ---- per-row metadata of the slice: 4 consecutive rows per thread --------
    // Only threads whose rows start inside the slice load, with one 16-byte
    // (scales, mask) or 4-byte (zero points) load per array when the base
    // pointers and the plane length keep those aligned (slices start on
    // multiples of 32 rows, so then the 4 rows never pass row S - 1); else row
    // by row, clamped.  Rows past the slice are loaded but never used.
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    const int r4 = tid * 4;
    const bool meta_live = r4 < n;
    const bool meta_vec = (a.S & 3) == 0 &&
                          (BLK || (((reinterpret_cast<uintptr_t>(a.ks) | reinterpret_cast<uintptr_t>(a.vs)) & 15) == 0 &&
                                   ((reinterpret_cast<uintptr_t>(a.kz) | reinterpret_cast<uintptr_t>(a.vz)) & 3) == 0)) &&
                          (!has_mask || ((reinterpret_cast<uintptr_t>(a.mask) & 15) == 0 && (a.mask_sb & 3) == 0));
    f32x4_t m_ks = {0.0f, 0.0f, 0.0f, 0.0f}, m_mk = m_ks, m_vs = m_ks;
    uint32_t m_kz = 0, m_vz = 0;
    if (meta_live) {
        const uint32_t j = (uint32_t)(j0 + r4);
        if (meta_vec) {
            if constexpr (!BLK) {
                m_ks = *(gptr<f32x4_t>)(ksb + j);
                m_vs = *(gptr<f32x4_t>)(vsb + j);
                m_kz = *(gptr<uint32_t>)(kzb + j);
                m_vz = *(gptr<uint32_t>)(vzb + j);
            }
            if (has_mask) m_mk = *(gptr<f32x4_t>)(mrow + j);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t je = (uint32_t)min((int)j + e, j1 - 1);
                if constexpr (!BLK) {
                    m_ks[e] = ksb[je];
                    m_vs[e] = vsb[je];
                    m_kz |= (uint32_t)(uint8_t)kzb[je] << (8 * e);
                    m_vz |= (uint32_t)(uint8_t)vzb[je] << (8 * e);
                }
                if (has_mask) m_mk[e] = mrow[je];
            }
        }
        if constexpr (BLK) {                         // scales live per block, applied in the passes
            m_ks = f32x4_t{1.0f, 1.0f, 1.0f, 1.0f};
            m_vs = m_ks;
        }
    }

    // K pass geometry: lane (rk, ck); rows j0 + (t * DEC_WAVES + wave) * RK + rk
    const int ck = lane % CK, rk = lane / CK;
    const int twk = n > wave * RK ? (n - wave * RK + STEPK - 1) / STEPK : 0;
    // V pass geometry: lane (rv, cv)
    const int cv = lane % CV, rv = lane / CV;
    const int twv = n > wave * RV ? (n - wave * RV + STEPV - 1) / STEPV : 0;

    auto krow = [&](int t) { return (uint32_t)min(j0 + (t * DEC_WAVES + wave) * RK + rk, j1 - 1); };
    auto vrow = [&](int t) { return (uint32_t)min(j0 + (t * DEC_WAVES + wave) * RV + rv, j1 - 1); };

    // ---- K ring: the first PD steps' codes go out before any arithmetic -------
    // Every slot is consumed (converted) before it is reloaded, so a reload
    // targets the same registers: a copy at the loop edge would wait for it.
    // Block caches: the scale of each 16-byte chunk's block rides in the ring
    // with the codes (16 bytes hold 16 FP8 or 32 FP4 elements, so a chunk
    // never straddles two 32-element blocks).
    uint4 kbuf[PD][KB / 16];
    uint32_t ksr[PD][KB / 16];
    auto fetch_codes = [&](int u, int t) {
        const uint32_t j = krow(t);
#pragma unroll
        for (int c = 0; c < KB / 16; ++c) {
            kbuf[u][c] = load16(kbase, j * ROWB + (uint32_t)ck * KB + 16 * c);
            if constexpr (BLK) {
                const uint32_t gi = j * SPR + (uint32_t)((ck * KB + 16 * c) * EPB) / 32;
                ksr[u][c] = SC8 ? (uint32_t)kscb[gi] : *(gptr<uint32_t>)(kscb + gi * SCB);
            }
        }
    };
#pragma unroll
    for (int u = 0; u < PD; ++u) fetch_codes(u, min(u, max(twk - 1, 0)));

    // ---- q in fp16, converted cooperatively; metadata into LDS ----------------
    // k = 0 when max|q| lies in [2^-8, 2^15); otherwise one power of two for
    // the G heads brings it into [2^14, 2^15).  A power-of-two rescale changes
    // no rounding, so both give the same result.
    float csc;        // sm_scale * log2(e) * 2^-k
    {
        float mx = 0.0f;
#pragma unroll
        for (int u = 0; u < QPT; ++u) mx = fmaxf(mx, fabsf(qv[u]));
        mx = wave_max(mx);
        if (lane == 0) s_red[wave][0] = mx;
        if (meta_live) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int zk = (int)(int8_t)(m_kz >> (8 * e)), zv = (int)(int8_t)(m_vz >> (8 * e));
                s_meta[r4 + e] = make_float4(m_ks[e], has_mask ? m_mk[e] * LOG2E : 0.0f, m_vs[e], (float)zv + VOFF);
                s_kzo[r4 + e] = zoff_pair(zk, U4);
            }
        }
        __syncthreads();
        mx = fmaxf(fmaxf(s_red[0][0], s_red[1][0]), fmaxf(s_red[2][0], s_red[3][0]));
        int k = 0;
        if (mx > 0.0f && !(mx >= 0x1p-8f && mx < 0x1p15f)) {
            int ex;
            frexpf(mx, &ex);
            k = 15 - ex;
        }
        csc = ldexpf(a.sm_scale_log2, -k);
        static_assert(QPT % 2 == 0, "q pairs");
#pragma unroll
        for (int u = 0; u < QPT; u += 2) {
            const int e = tid * QPT + u;
            if (e < NQ) {
                const float x0 = ldexpf(qv[u], k), x1 = ldexpf(qv[u + 1], k);
                const _Float16 h0v = (_Float16)x0, h1v = (_Float16)x1;
                half2_t hv = {h0v, h1v};
                const int hh = e / D, pr = (e % D) / 2;
                s_q[hh][0][pr] = __builtin_bit_cast(uint32_t, hv);
                if constexpr (NL == 2) {
                    half2_t lv = {(_Float16)(x0 - (float)h0v), (_Float16)(x1 - (float)h1v)};
                    s_q[hh][NL - 1][pr] = __builtin_bit_cast(uint32_t, lv);
                }
            }
        }
    }
    __syncthreads();                                  // s_q, s_meta, s_kzo ready
    uint32_t qh[G][NL][NPK];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int l2 = 0; l2 < NL; ++l2)
#pragma unroll
            for (int i = 0; i < NPK; ++i) qh[hh][l2][i] = s_q[hh][l2][ck * NPK + i];

    // ---- pass 1: q . (code - zp) per row into LDS -----------------------------
    auto k_step = [&](int u, int t, bool reload) {
        const int i = (t * DEC_WAVES + wave) * RK + rk;
        constexpr int NC = KB / 16, PPC = NPK / NC;   // 16-byte chunks, fp16 pairs per chunk
        uint32_t kh[NPK];
        float kscale[NC];
        if constexpr (BLK) {
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                blk_to_h2<QM>(kbuf[u][c], kh + c * PPC);
                kscale[c] = blk_scale<SC8>(ksr[u][c]);
            }
        } else {
            const uint32_t zo = s_kzo[min(i, i_last)];
#pragma unroll
            for (int c = 0; c < NC; ++c) codes_to_h2<U4>(kbuf[u][c], zo, kh + c * PPC);
        }
        if (reload) {
            __builtin_amdgcn_sched_barrier(0);        // keep the reload after the conversion
            fetch_codes(u, min(t + PD, twk - 1));
        }
        float d[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            float x;
            if constexpr (BLK) {
                // per chunk: q . codes, times the chunk's block scale
                x = 0.0f;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    float xc = 0.0f;
#pragma unroll
                    for (int e = c * PPC; e < (c + 1) * PPC; ++e) {
                        xc = __builtin_amdgcn_fdot2(as_h2(qh[hh][0][e]), as_h2(kh[e]), xc, false);
                        if constexpr (NL == 2) xc = __builtin_amdgcn_fdot2(as_h2(qh[hh][1][e]), as_h2(kh[e]), xc, false);
                    }
                    x = fmaf(xc, kscale[c], x);
                }
            } else {
                x = __builtin_amdgcn_fdot2(as_h2(qh[hh][0][0]), as_h2(kh[0]), 0.0f, false);
                if constexpr (NL == 2) x = __builtin_amdgcn_fdot2(as_h2(qh[hh][1][0]), as_h2(kh[0]), x, false);
#pragma unroll
                for (int e = 1; e < NPK; ++e) {
                    x = __builtin_amdgcn_fdot2(as_h2(qh[hh][0][e]), as_h2(kh[e]), x, false);
                    if constexpr (NL == 2) x = __builtin_amdgcn_fdot2(as_h2(qh[hh][1][e]), as_h2(kh[e]), x, false);
                }
            }
            d[hh] = group_sum_first<CK>(x);
        }
        if (ck == 0 && i < n) {
#pragma unroll
            for (int hh = 0; hh < G; ++hh) s_row[i * G + hh] = d[hh];
        }
    };
    int t0 = 0;
    for (; t0 + PD <= twk; t0 += PD) {               // whole ring rounds
#pragma unroll
        for (int u = 0; u < PD; ++u) k_step(u, t0 + u, true);
    }
#pragma unroll
    for (int u = 0; u < PD - 1; ++u)                 // the rest: already in the ring
        if (t0 + u < twk) k_step(u, t0 + u, false);

    // ---- V ring: the first PDV steps go out before the barrier, so the V
    // stream runs while the middle pass computes
    uint4 vbuf[PDV];
    uint32_t vsr[PDV];                                // block caches: the chunk's block scale
    auto fetch_v = [&](int u, int t) {
        const uint32_t j = vrow(t);
        vbuf[u] = load16(vbase, j * ROWB + (uint32_t)cv * 16);
        if constexpr (BLK) {
            const uint32_t gi = j * SPR + (uint32_t)(cv * 16 * EPB) / 32;
            vsr[u] = SC8 ? (uint32_t)vscb[gi] : *(gptr<uint32_t>)(vscb + gi * SCB);
        }
    };
#pragma unroll
    for (int u = 0; u < PDV; ++u) fetch_v(u, min(u, max(twv - 1, 0)));
    __syncthreads();                                  // all dots in LDS

    // ---- middle pass: per head, scores, max, p * scale_v, l, zp correction ----
    // wave w owns heads [(w / WPH) * HPW, + HPW) and rows (w % WPH) * 64 + lane
    // + 64 * WPH * u of the slice
    constexpr int WPH = DEC_WAVES / G >= 1 ? DEC_WAVES / G : 1;   // waves per head
    constexpr int HPW = G / DEC_WAVES >= 1 ? G / DEC_WAVES : 1;   // heads per wave
    {
        // rows go in groups of MB per lane: the LDS reads of a group are issued
        // together (clamped to the last row; rows past the slice are masked)
        constexpr int MB = 4;
        constexpr int RS = 64 * WPH;                  // row stride between a lane's rows
        const int h_first = (wave / WPH) * HPW;
        const int r_first = (wave % WPH) * 64 + lane;
        float mloc[HPW];
#pragma unroll
        for (int hx = 0; hx < HPW; ++hx) mloc[hx] = NEG_INF;
        for (int i0 = r_first; i0 < n; i0 += MB * RS) {
            float2 mt[MB];
            float dv[MB][HPW];
#pragma unroll
            for (int u = 0; u < MB; ++u) {
                const int ii = min(i0 + u * RS, i_last);
                const float4 m4 = s_meta[ii];
                mt[u] = make_float2(m4.x * csc, m4.y);
#pragma unroll
                for (int hx = 0; hx < HPW; ++hx) dv[u][hx] = s_row[ii * G + h_first + hx];
            }
#pragma unroll
            for (int u = 0; u < MB; ++u) {
                const int i = i0 + u * RS;
                if (i < n) {
#pragma unroll
                    for (int hx = 0; hx < HPW; ++hx) {
                        // a masked row is -inf whatever its (possibly unwritten) scale holds
                        const float sc = mt[u].y == NEG_INF ? NEG_INF : fmaf(dv[u][hx], mt[u].x, mt[u].y);
                        s_row[i * G + h_first + hx] = sc;
                        mloc[hx] = fmaxf(mloc[hx], sc);
                    }
                }
            }
        }
        float msafe[HPW];
#pragma unroll
        for (int hx = 0; hx < HPW; ++hx) {
            float mm = wave_max(mloc[hx]);
            if constexpr (WPH > 1) {
                if (lane == 0) s_red[wave][hx] = mm;
                __syncthreads();
                mm = NEG_INF;
#pragma unroll
                for (int w = 0; w < WPH; ++w) mm = fmaxf(mm, s_red[(wave / WPH) * WPH + w][hx]);
                __syncthreads();
            }
            if ((wave % WPH) == 0 && lane == 0) s_mx[h_first + hx] = mm;
            msafe[hx] = mm == NEG_INF ? 0.0f : mm;
        }
        float lsum[HPW], csum[HPW];
#pragma unroll
        for (int hx = 0; hx < HPW; ++hx) { lsum[hx] = 0.0f; csum[hx] = 0.0f; }
        for (int i0 = r_first; i0 < n; i0 += MB * RS) {
            float2 mt[MB];
            float sv[MB][HPW];
#pragma unroll
            for (int u = 0; u < MB; ++u) {
                const int ii = min(i0 + u * RS, i_last);
                const float4 m4 = s_meta[ii];
                mt[u] = make_float2(m4.z, m4.w);
#pragma unroll
                for (int hx = 0; hx < HPW; ++hx) sv[u][hx] = s_row[ii * G + h_first + hx];
            }
#pragma unroll
            for (int u = 0; u < MB; ++u) {
                const int i = i0 + u * RS;
                if (i < n) {
#pragma unroll
                    for (int hx = 0; hx < HPW; ++hx) {
                        const float p = __builtin_amdgcn_exp2f(sv[u][hx] - msafe[hx]);
                        const float pv = p == 0.0f ? 0.0f : p * mt[u].x;   // a dropped row adds exactly 0
                        lsum[hx] += p;
                        csum[hx] = fmaf(pv, mt[u].y, csum[hx]);
                        s_row[i * G + h_first + hx] = pv;
                    }
                }
            }
        }
#pragma unroll
        for (int hx = 0; hx < HPW; ++hx) {
            const float lw = wave_sum(lsum[hx]), cw = wave_sum(csum[hx]);
            if (lane == 0) { s_red[wave][hx] = lw; s_o[wave][hx][0] = cw; }
        }
    }
    __syncthreads();                                  // p * scale_v and per-wave sums ready
    if (tid < G) {
        const int w0 = (tid / HPW) * WPH, hx = tid % HPW;
        float lv = 0.0f, cvv = 0.0f;
#pragma unroll
        for (int w = 0; w < WPH; ++w) { lv += s_red[w0 + w][hx]; cvv += s_o[w0 + w][hx][0]; }
        s_l[tid] = lv;
        s_corr[tid] = cvv;
    }

    // ---- pass 2: acc += (p * scale_v) * (code + VOFF) ---------------------------
    float acc[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) acc[e] = 0.0f;
    auto v_step = [&](int u, int t, bool reload) {
        float vf[EV];
        float live_sc = 1.0f;
        if constexpr (BLK) {
            blk_to_f32<QM>(vbuf[u], vf);
            live_sc = blk_scale<SC8>(vsr[u]);
        } else {
            codes_to_f32<U4>(vbuf[u], vf);
        }
        if (reload) {
            __builtin_amdgcn_sched_barrier(0);        // keep the reload after the conversion
            fetch_v(u, min(t + PDV, twv - 1));
        }
        // rows past the slice read the last row (finite) and weigh it by 0
        const int i = (t * DEC_WAVES + wave) * RV + rv;
        const float live = i < n ? live_sc : 0.0f;
        const int ic = min(i, i_last);
        float pv[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const float w = s_row[ic * G + hh];
            pv[hh] = w == 0.0f ? 0.0f : w * live;      // a dropped row adds exactly 0, whatever its scale
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
#pragma unroll
            for (int e = 0; e < EV; ++e) acc[hh * EV + e] = fmaf(pv[hh], vf[e], acc[hh * EV + e]);
    };
    t0 = 0;
    for (; t0 + PDV <= twv; t0 += PDV) {
#pragma unroll
        for (int u = 0; u < PDV; ++u) v_step(u, t0 + u, true);
    }
#pragma unroll
    for (int u = 0; u < PDV - 1; ++u)
        if (t0 + u < twv) v_step(u, t0 + u, false);

    // ---- merge: row groups (reduce-scatter), then waves, then the partial -------
    reduce_scatter<NV, 32, CV>(acc, lane);
    __syncthreads();                                  // s_o (used for sums above) free again
#pragma unroll
    for (int e = 0; e < NVR; ++e) {
        const int v = rv * NVR + e;                    // head v / EV, element v % EV
        s_o[wave][v / EV][cv * EV + v % EV] = acc[e];
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += 256) {
        const int hh = idx / D, d = idx % D;
        float o = 0.0f;
#pragma unroll
        for (int w = 0; w < DEC_WAVES; ++w) o += s_o[w][hh][d];
        const int64_t ph = ((int64_t)b * a.Hq + g * G + hh) * nsplit + split;
        a.part_o[ph * D + d] = o - s_corr[hh];
        if (d == 0) {
            a.part_ml[ph * 2] = s_mx[hh];
            a.part_ml[ph * 2 + 1] = s_l[hh];
        }
    }
}

// Merge the splits of one row -- a (b, query head) of decode, a (b, query
// head, query row) of a key-split prefill: o = sum_s o_s 2^(m_s - m*) / l
// with l = sum_s l_s 2^(m_s - m*).  The splits go in chunks of CH whose o and
// (m, l) loads are all issued before any arithmetic (one memory round trip
// per chunk); a running maximum rescales the sums between chunks.  A row
// with no visible key (every m_s = -inf) gives 0.
template <int D>
__global__ __launch_bounds__(D) void sdpa_decode_combine(const float* __restrict__ part_o,
                                                         const float* __restrict__ part_ml, int nsplit,
                                                         void* __restrict__ out, int out_bf16) {
    constexpr int CH = 16;
    constexpr float NEG_INF = -__builtin_huge_valf();
    const int64_t bh = blockIdx.x;
    const int d = threadIdx.x;
    const gptr<float> po = uniform_ptr(part_o + bh * nsplit * D);
    const gptr<float> pml = uniform_ptr(part_ml + bh * nsplit * 2);
    float m = NEG_INF, l = 0.0f, acc = 0.0f;
    for (int s0 = 0; s0 < nsplit; s0 += CH) {
        float mv[CH], lv[CH], ov[CH];
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            const uint32_t sp = (uint32_t)min(s0 + u, nsplit - 1);
            mv[u] = pml[2 * sp];
            lv[u] = pml[2 * sp + 1];
            ov[u] = po[sp * D + d];
        }
        __builtin_amdgcn_sched_barrier(0);            // every load of the chunk is issued first
        float mn = m;
#pragma unroll
        for (int u = 0; u < CH; ++u)
            if (s0 + u < nsplit) mn = fmaxf(mn, mv[u]);
        const float r = m == NEG_INF ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
        acc *= r;
        l *= r;
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            const bool live = s0 + u < nsplit && mv[u] != NEG_INF;
            const float w = live ? __builtin_amdgcn_exp2f(mv[u] - mn) : 0.0f;
            acc = fmaf(w, ov[u], acc);
            l = fmaf(w, lv[u], l);
        }
        m = mn;
    }
    const float res = l > 0.0f ? acc / l : 0.0f;
    if (out_bf16) reinterpret_cast<uint16_t*>(out)[bh * D + d] = f32_to_bf16_rne(res);
    else reinterpret_cast<float*>(out)[bh * D + d] = res;
}

// Upper bound on the split count (sizes the workspace without a device):
// enough splits for 4096 resident workgroups, and at least enough that every
// slice fits the LDS row buffer.
int decode_splits_max(int B, int Hq, int Hkv, int S, int D, int qmode) {
    const DecGeom gm = dec_geom(D, qmode == QM_UINT4_TH || qmode == QM_MXFP4_B32 || qmode == QM_MXFP4E1M2_B32, Hq / Hkv);
    const int pairs = B * Hkv;
    const int max_useful = (S + DEC_CHUNK_ALIGN - 1) / DEC_CHUNK_ALIGN;
    int splits = (4096 + pairs - 1) / pairs;
    if (splits > max_useful) splits = max_useful;
    const int need = (S + gm.rows_max - 1) / gm.rows_max;   // ceil(S / splits) <= rows_max
    return splits > need ? splits : need;
}

template <int D, int QM, int G, bool QBF16>
static const void* split_kernel() { return reinterpret_cast<const void*>(&sdpa_decode_split<D, QM, G, QBF16>); }

static const void* split_kernel_for(int D, int qm, int G, bool qbf16) {
#define KVQ_SK(DD, QQ)                                                                          \
    switch (G) {                                                                                \
    case 1: return qbf16 ? split_kernel<DD, QQ, 1, true>() : split_kernel<DD, QQ, 1, false>(); \
    case 2: return qbf16 ? split_kernel<DD, QQ, 2, true>() : split_kernel<DD, QQ, 2, false>(); \
    case 4: return qbf16 ? split_kernel<DD, QQ, 4, true>() : split_kernel<DD, QQ, 4, false>(); \
    default: return qbf16 ? split_kernel<DD, QQ, 8, true>() : split_kernel<DD, QQ, 8, false>(); \
    }
#define KVQ_SKD(DD)                                          \
    switch (qm) {                                            \
    case QM_INT8_TH: { KVQ_SK(DD, QM_INT8_TH) }              \
    case QM_UINT4_TH: { KVQ_SK(DD, QM_UINT4_TH) }            \
    case QM_FP8E4M3_B32: { KVQ_SK(DD, QM_FP8E4M3_B32) }      \
    case QM_MXFP8_B32: { KVQ_SK(DD, QM_MXFP8_B32) }          \
    case QM_FP8E5M2_B32: { KVQ_SK(DD, QM_FP8E5M2_B32) }      \
    case QM_INT8_B32: { KVQ_SK(DD, QM_INT8_B32) }            \
    case QM_MXFP4E1M2_B32: { KVQ_SK(DD, QM_MXFP4E1M2_B32) }  \
    default: { KVQ_SK(DD, QM_MXFP4_B32) }                    \
    }
    if (D == 64) { KVQ_SKD(64) }
    if (D == 128) { KVQ_SKD(128) }
    KVQ_SKD(256)
#undef KVQ_SKD
#undef KVQ_SK
}

// Workgroups of one split-kernel instantiation to keep on the device at once:
// per CU, the smaller of the VGPR limit (512 registers per lane of a SIMD in
// granules of 8; a 4-wave workgroup puts one wave on each SIMD), the LDS limit
// and 2, times the CU count.  0 when the runtime cannot tell.  Two per CU
// (8 waves) ran as fast as three or faster on the int8 decode at batch 1 to 32
// and 1k to 32k keys (up to 15-20% at batch 1-4): each workgroup's prologue,
// merge and partials cost more than a third workgroup's latency hiding buys.
// Counts that leave CUs unevenly loaded (between two and three per CU) were
// slower than either.
static int resident_workgroups(int D, int qm, int G, bool qbf16) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    const int key = ((D == 64 ? 0 : D == 128 ? 1 : 2) * 8 + (qm & 7)) * 8 + (G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3) * 2 +
                    (qbf16 ? 1 : 0);
    static int cache[64][192];                        // 0 = not known yet; benign races
    int v = cache[dev][key];
    if (v > 0) return v;
    hipFuncAttributes fa;
    int cus = 0, lds_cu = 0;
    if (hipFuncGetAttributes(&fa, split_kernel_for(D, qm, G, qbf16)) != hipSuccess || fa.numRegs <= 0 ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
        lds_cu <= 0)
        lds_cu = 160 * 1024;
    const int granule = (fa.numRegs + 7) / 8 * 8;
    int per_cu = 512 / granule;
    if (per_cu > 2) per_cu = 2;
    if (fa.sharedSizeBytes > 0) {
        const int by_lds = lds_cu / (int)fa.sharedSizeBytes;
        if (by_lds < per_cu) per_cu = by_lds;
    }
    if (per_cu < 1) per_cu = 1;
    v = per_cu * cus;
    cache[dev][key] = v;
    return v;
}

// Split count of a launch: as many splits as keep every workgroup resident in
// one round (a second, partly filled round would run with little latency
// hiding), within [rows fit in LDS, decode_splits_max].
int decode_splits(int B, int Hq, int Hkv, int S, int D, int qmode, bool qbf16) {
    const DecGeom gm = dec_geom(D, qmode == QM_UINT4_TH || qmode == QM_MXFP4_B32 || qmode == QM_MXFP4E1M2_B32, Hq / Hkv);
    const int pairs = B * Hkv;
    const int hi = decode_splits_max(B, Hq, Hkv, S, D, qmode);
    const int need = (S + gm.rows_max - 1) / gm.rows_max;
    int resident = resident_workgroups(D, qmode, Hq / Hkv, qbf16);
    if (resident <= 0) resident = 1024;
    int splits = resident / pairs;
    if (splits < need) splits = need;
    if (splits > hi) splits = hi;
    return splits < 1 ? 1 : splits;
}

template <int D, int QM, int G, bool QBF16>
static hipError_t launch_split(const DecodeArgs& a, int nsplit, hipStream_t s) {
    const dim3 grid(nsplit, a.Hkv, a.B);
    hipLaunchKernelGGL((sdpa_decode_split<D, QM, G, QBF16>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int D, int QM, bool QBF16>
static hipError_t dispatch_g(const DecodeArgs& a, int G, int nsplit, hipStream_t s) {
    switch (G) {
    case 1: return launch_split<D, QM, 1, QBF16>(a, nsplit, s);
    case 2: return launch_split<D, QM, 2, QBF16>(a, nsplit, s);
    case 4: return launch_split<D, QM, 4, QBF16>(a, nsplit, s);
    case 8: return launch_split<D, QM, 8, QBF16>(a, nsplit, s);
    default: return hipErrorInvalidValue;
    }
}

template <int D, int QM>
static hipError_t dispatch_q(const DecodeArgs& a, bool qbf16, int G, int nsplit, hipStream_t s) {
    return qbf16 ? dispatch_g<D, QM, true>(a, G, nsplit, s) : dispatch_g<D, QM, false>(a, G, nsplit, s);
}

template <int D>
static hipError_t dispatch_m(const DecodeArgs& a, int qmode, bool qbf16, int G, int nsplit, hipStream_t s) {
    switch (qmode) {
    case QM_INT8_TH: return dispatch_q<D, QM_INT8_TH>(a, qbf16, G, nsplit, s);
    case QM_UINT4_TH: return dispatch_q<D, QM_UINT4_TH>(a, qbf16, G, nsplit, s);
    case QM_FP8E4M3_B32: return dispatch_q<D, QM_FP8E4M3_B32>(a, qbf16, G, nsplit, s);
    case QM_MXFP4_B32: return dispatch_q<D, QM_MXFP4_B32>(a, qbf16, G, nsplit, s);
    case QM_MXFP8_B32: return dispatch_q<D, QM_MXFP8_B32>(a, qbf16, G, nsplit, s);
    case QM_FP8E5M2_B32: return dispatch_q<D, QM_FP8E5M2_B32>(a, qbf16, G, nsplit, s);
    case QM_INT8_B32: return dispatch_q<D, QM_INT8_B32>(a, qbf16, G, nsplit, s);
    case QM_MXFP4E1M2_B32: return dispatch_q<D, QM_MXFP4E1M2_B32>(a, qbf16, G, nsplit, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_sdpa_decode(const DecodeLaunch& L, hipStream_t s) {
    DecodeArgs a{L.q, L.B, L.Hq, L.Hkv, L.S, L.kc, L.ks, L.kz, L.vc, L.vs, L.vz, L.kv_len, L.kv_len_sb,
                 L.mask, L.mask_sb, L.sm_scale * 1.4426950408889634f, L.part_o, L.part_ml, L.err};
    const int G = L.Hq / L.Hkv;
    hipError_t e;
    switch (L.D) {
    case 64: e = dispatch_m<64>(a, L.qmode, L.q_bf16, G, L.nsplit, s); break;
    case 128: e = dispatch_m<128>(a, L.qmode, L.q_bf16, G, L.nsplit, s); break;
    case 256: e = dispatch_m<256>(a, L.qmode, L.q_bf16, G, L.nsplit, s); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    return launch_split_combine(L.D, L.part_o, L.part_ml, L.nsplit, (int64_t)L.B * L.Hq, L.out, L.out_bf16, s);
}

hipError_t launch_split_combine(int D, const float* part_o, const float* part_ml, int nsplit, int64_t rows,
                                void* out, bool out_bf16, hipStream_t s) {
    if (rows <= 0 || rows > 0x7FFFFFFF) return hipErrorInvalidValue;
    const unsigned nr = (unsigned)rows;
    const int ob = out_bf16 ? 1 : 0;
    switch (D) {
    case 64: hipLaunchKernelGGL((sdpa_decode_combine<64>), dim3(nr), dim3(64), 0, s, part_o, part_ml, nsplit, out, ob); break;
    case 128: hipLaunchKernelGGL((sdpa_decode_combine<128>), dim3(nr), dim3(128), 0, s, part_o, part_ml, nsplit, out, ob); break;
    case 256: hipLaunchKernelGGL((sdpa_decode_combine<256>), dim3(nr), dim3(256), 0, s, part_o, part_ml, nsplit, out, ob); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kvq
