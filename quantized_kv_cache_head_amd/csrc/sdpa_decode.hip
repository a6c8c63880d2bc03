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
//  * grid (splits, Hkv, B); a 256-thread workgroup owns one (b, kv head g)
//    and one contiguous slice of [0, kv_len) whose length is derived on the
//    device from kv_len, so the launch shape is fixed across steps.
//  * The G = Hq/Hkv query heads of a KV head are processed together: every
//    K/V byte is read from HBM once for all of them.
//  * A KV row of ROWB bytes is split over C = ROWB/16 lanes, 16 bytes per
//    lane (one dwordx4 load for K, one for V); a wave covers R = 64/C rows
//    per step and the 4 waves of the workgroup read adjacent rows.
//  * q . k: codes become exact fp16 integers (code - zp) (a byte permute under
//    the fp16 exponent of 1024, then one packed fp16 subtraction) and are
//    multiplied with q (rescaled by a power of two into fp16 range; exact for
//    bf16 q) by v_dot2_f32_f16 with fp32 accumulation.  fp32 q uses a hi + lo
//    pair of fp16 limbs.
//  * p . v: fp32 FMA on v_cvt_f32_ubyte of the codes; p is folded with the
//    row's scale, the zero point and offset are removed through one running
//    correction per head.
//  * Each lane keeps an online softmax (m, l) for its row group.  Rows go in
//    blocks of NB steps: the K and V loads of a block are issued together
//    (bytes in flight without extra waves), the block's scores stay in
//    registers, the running max moves once per block (one unconditional
//    rescale, no data-dependent branch), then p * v is accumulated; the
//    row groups, then the waves, are
//    merged at the end (common max, then a reduce-scatter of the
//    accumulators with lane-swap permutes) and one partial (m, l, o[D]) per
//    (b, head, split) goes to the workspace; a small combine kernel merges the
//    splits (a separate launch: merging inside the split kernel would need a
//    device-scope release/acquire per workgroup, which on this multi-XCD part
//    writes back and invalidates L2).
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
    const float* mask;
    int64_t mask_sb;
    float sm_scale_log2;   // sm_scale * log2(e)
    float* part_o;         // [B, Hq, splits, D]
    float* part_ml;        // [B, Hq, splits, 2]
    int32_t* err;
};

constexpr int DEC_WAVES = 4;
constexpr float LAZY_TAU = 8.0f;   // rescale threshold in log2 units

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
    int rowb, kb, ck, rk, cv, rv, stepk, stepv, stepm, rows_max;
};
__host__ __device__ constexpr DecGeom dec_geom(int D, bool u4, int G) {
    const int rowb = u4 ? D / 2 : D;
    const int kb = (G * 32 * (u4 ? 2 : 1) <= 128 && rowb >= 64) ? 32 : 16;
    const int ck = rowb / kb, rk = 64 / ck;
    const int cv = rowb / 16, rv = 64 / cv;
    const int stepk = rk * DEC_WAVES, stepv = rv * DEC_WAVES;
    const int rows_max = 4096 / G < 1024 ? 4096 / G : 1024;
    return DecGeom{rowb, kb, ck, rk, cv, rv, stepk, stepv, stepk > stepv ? stepk : stepv, rows_max};
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

template <int D, bool U4, int G, bool QBF16>
__global__ __launch_bounds__(256) void sdpa_decode_split(DecodeArgs a) {
    constexpr DecGeom GM = dec_geom(D, U4, G);
    constexpr int ROWB = GM.rowb;
    constexpr int EPB = U4 ? 2 : 1;                  // elements per code byte
    constexpr int KB = GM.kb, CK = GM.ck, RK = GM.rk;
    constexpr int NPK = KB * EPB / 2;                // fp16 pairs per lane, K pass
    constexpr int CV = GM.cv, RV = GM.rv;
    constexpr int EV = 16 * EPB;                     // elements per lane, V pass
    constexpr int NL = QBF16 ? 1 : 2;                // fp16 limbs of q
    constexpr float VOFF = U4 ? 0.0f : 128.0f;      // fp32 value = code + VOFF
    constexpr int NV = G * EV;                       // accumulators per lane
    constexpr int NVR = NV / RV;                     // after the row-group reduce-scatter
    constexpr int STEPK = GM.stepk, STEPV = GM.stepv, STEPM = GM.stepm;
    constexpr int PD = KVQ_DEC_PD;                   // ring depth (steps in flight)
    constexpr int ROWS_MAX = GM.rows_max;
    constexpr float NEG_INF = -__builtin_huge_valf();
    constexpr float LOG2E = 1.4426950408889634f;
    static_assert(CK >= 1 && CK <= 16 && CV >= 2 && CV <= 16, "row split");
    static_assert(ROWS_MAX % STEPM == 0, "rows_max must hold whole steps");

    __shared__ float s_row[ROWS_MAX * G];           // scores, then p * scale_v
    __shared__ float2 s_meta[ROWS_MAX];             // (scale_v, zp_v + VOFF) per row
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
    int kv_len = a.kv_len ? *a.kv_len : a.S;
    if (kv_len < 1 || kv_len > a.S) {
        if (a.err && split == 0 && g == 0 && b == 0 && tid == 0) atomicOr(a.err, KVQ_DEV_FLAG_KVLEN);
        kv_len = kv_len < 1 ? 1 : a.S;
    }
    int chunk = (kv_len + nsplit - 1) / nsplit;
    chunk = (chunk + STEPM - 1) / STEPM * STEPM;    // <= ROWS_MAX by the host's split count
    const int j0 = split * chunk;
    const int j1 = min(j0 + chunk, kv_len);          // j1 - 1 is a valid row even when empty
    const int n = max(j1 - j0, 0);

    const int64_t plane = ((int64_t)b * a.Hkv + g) * a.S;
    const gptr<uint8_t> kbase = uniform_ptr(a.kc + plane * ROWB);
    const gptr<uint8_t> vbase = uniform_ptr(a.vc + plane * ROWB);
    const gptr<float> ksb = uniform_ptr(a.ks + plane);
    const gptr<float> vsb = uniform_ptr(a.vs + plane);
    const gptr<int8_t> kzb = uniform_ptr(a.kz + plane);
    const gptr<int8_t> vzb = uniform_ptr(a.vz + plane);
    const bool has_mask = a.mask != nullptr;
    // without a mask the mask load reads the key scales (any valid row) and
    // its value is dropped
    const gptr<float> mrow = has_mask ? uniform_ptr(a.mask + (int64_t)b * a.mask_sb) : ksb;

    // K pass geometry: lane (rk, ck); rows j0 + (t * DEC_WAVES + wave) * RK + rk
    const int ck = lane % CK, rk = lane / CK;
    const int twk = n > wave * RK ? (n - wave * RK + STEPK - 1) / STEPK : 0;
    // V pass geometry: lane (rv, cv)
    const int cv = lane % CV, rv = lane / CV;
    const int twv = n > wave * RV ? (n - wave * RV + STEPV - 1) / STEPV : 0;

    auto krow = [&](int t) { return (uint32_t)min(j0 + (t * DEC_WAVES + wave) * RK + rk, j1 - 1); };
    auto vrow = [&](int t) { return (uint32_t)min(j0 + (t * DEC_WAVES + wave) * RV + rv, j1 - 1); };

    // ---- K ring: codes and per-row metadata of PD steps ---------------------
    // Every slot is consumed before it is reloaded (codes after their
    // conversion, metadata after the step's LDS stores), so a reload targets
    // the same registers: a copy at the loop edge would wait for the load.
    uint4 kbuf[PD][KB / 16];
    int kzr[PD], vzr[PD];
    float ksr[PD], mkr[PD], vsr[PD];
    auto fetch_codes = [&](int u, int t) {
        const uint32_t j = krow(t);
#pragma unroll
        for (int c = 0; c < KB / 16; ++c) kbuf[u][c] = load16(kbase, j * ROWB + (uint32_t)ck * KB + 16 * c);
    };
    auto fetch_meta = [&](int u, int t) {
        const uint32_t j = krow(t);
        kzr[u] = kzb[j];
        ksr[u] = ksb[j];
        mkr[u] = mrow[j];
        vsr[u] = vsb[j];
        vzr[u] = vzb[j];
    };
#pragma unroll
    for (int u = 0; u < PD; ++u) {
        fetch_codes(u, min(u, max(twk - 1, 0)));
        fetch_meta(u, min(u, max(twk - 1, 0)));
    }

    // ---- q in fp16, converted cooperatively --------------------------------
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
    __syncthreads();                                  // s_q ready
    uint32_t qh[G][NL][NPK];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int l2 = 0; l2 < NL; ++l2)
#pragma unroll
            for (int i = 0; i < NPK; ++i) qh[hh][l2][i] = s_q[hh][l2][ck * NPK + i];

    // ---- pass 1: scores (log2 units, mask added) and V metadata into LDS -----
    // Steps past this wave's rows run on clamped rows and store nothing.
    for (int t0 = 0; t0 < twk; t0 += PD) {
#pragma unroll
        for (int u = 0; u < PD; ++u) {
            const int t = t0 + u;
            uint32_t kh[NPK];
            const uint32_t zo = zoff_pair(kzr[u], U4);
#pragma unroll
            for (int c = 0; c < KB / 16; ++c) codes_to_h2<U4>(kbuf[u][c], zo, kh + c * (NPK / (KB / 16)));
            __builtin_amdgcn_sched_barrier(0);      // keep the reload after the conversion
            fetch_codes(u, min(t + PD, twk - 1));
            float d[G];
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                float x = __builtin_amdgcn_fdot2(as_h2(qh[hh][0][0]), as_h2(kh[0]), 0.0f, false);
                if constexpr (NL == 2) x = __builtin_amdgcn_fdot2(as_h2(qh[hh][1][0]), as_h2(kh[0]), x, false);
#pragma unroll
                for (int i = 1; i < NPK; ++i) {
                    x = __builtin_amdgcn_fdot2(as_h2(qh[hh][0][i]), as_h2(kh[i]), x, false);
                    if constexpr (NL == 2) x = __builtin_amdgcn_fdot2(as_h2(qh[hh][1][i]), as_h2(kh[i]), x, false);
                }
                d[hh] = group_sum_first<CK>(x);
            }
            const int i = (t * DEC_WAVES + wave) * RK + rk;
            if (ck == 0 && i < n) {
                const float ks = ksr[u] * csc;
                const float madd = has_mask ? mkr[u] * LOG2E : 0.0f;
#pragma unroll
                for (int hh = 0; hh < G; ++hh) s_row[i * G + hh] = fmaf(d[hh], ks, madd);
                s_meta[i] = make_float2(vsr[u], (float)vzr[u] + VOFF);
            }
            __builtin_amdgcn_sched_barrier(0);
            fetch_meta(u, min(t + PD, twk - 1));
        }
    }

    // ---- V ring: the first loads go out before the barrier --------------------
    uint4 vbuf[PD];
#pragma unroll
    for (int u = 0; u < PD; ++u)
        vbuf[u] = load16(vbase, vrow(min(u, max(twv - 1, 0))) * ROWB + (uint32_t)cv * 16);
    __syncthreads();                                  // all scores in LDS

    // ---- middle pass: per head, max, p * scale_v, l, zero-point correction ----
    // wave w owns heads [(w / WPH) * HPW, + HPW) and rows (w % WPH) * 64 + lane
    // + 64 * WPH * u of the slice
    constexpr int WPH = DEC_WAVES / G >= 1 ? DEC_WAVES / G : 1;   // waves per head
    constexpr int HPW = G / DEC_WAVES >= 1 ? G / DEC_WAVES : 1;   // heads per wave
    {
        const int h_first = (wave / WPH) * HPW;
        const int r_first = (wave % WPH) * 64 + lane;
        float mloc[HPW];
#pragma unroll
        for (int hx = 0; hx < HPW; ++hx) mloc[hx] = NEG_INF;
        for (int i = r_first; i < n; i += 64 * WPH) {
#pragma unroll
            for (int hx = 0; hx < HPW; ++hx) mloc[hx] = fmaxf(mloc[hx], s_row[i * G + h_first + hx]);
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
        for (int i = r_first; i < n; i += 64 * WPH) {
            const float2 mt = s_meta[i];
#pragma unroll
            for (int hx = 0; hx < HPW; ++hx) {
                const int hh = h_first + hx;
                const float p = __builtin_amdgcn_exp2f(s_row[i * G + hh] - msafe[hx]);
                const float pv = p * mt.x;
                lsum[hx] += p;
                csum[hx] = fmaf(pv, mt.y, csum[hx]);
                s_row[i * G + hh] = pv;
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
    // Steps past the slice read a clamped LDS row and use p = 0.
    float acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = 0.0f;
    const int i_last = max(n - 1, 0);
    for (int t0 = 0; t0 < twv; t0 += PD) {
#pragma unroll
        for (int u = 0; u < PD; ++u) {
            const int t = t0 + u;
            float vf[EV];
            codes_to_f32<U4>(vbuf[u], vf);
            __builtin_amdgcn_sched_barrier(0);      // keep the reload after the conversion
            vbuf[u] = load16(vbase, vrow(min(t + PD, twv - 1)) * ROWB + (uint32_t)cv * 16);
            // rows past the slice read the last row (finite) and weigh it by 0
            const int i = (t * DEC_WAVES + wave) * RV + rv;
            const float live = i < n ? 1.0f : 0.0f;
            const int ic = min(i, i_last);
            float pv[G];
#pragma unroll
            for (int hh = 0; hh < G; ++hh) pv[hh] = s_row[ic * G + hh] * live;
#pragma unroll
            for (int hh = 0; hh < G; ++hh)
#pragma unroll
                for (int e = 0; e < EV; ++e) acc[hh * EV + e] = fmaf(pv[hh], vf[e], acc[hh * EV + e]);
        }
    }

    // ---- merge: row groups (reduce-scatter), then waves, then the partial -------
    reduce_scatter<NV, 32, CV>(acc, lane);
    __syncthreads();                                  // s_o (used for sums above) free again
#pragma unroll
    for (int i = 0; i < NVR; ++i) {
        const int v = rv * NVR + i;                    // head v / EV, element v % EV
        s_o[wave][v / EV][cv * EV + v % EV] = acc[i];
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

// Merge the splits of one (b, query head): o = sum_s o_s 2^(m_s - m*) / l.
// The (m, l) pairs go through LDS once; the o loads are independent.
template <int D>
__global__ __launch_bounds__(D) void sdpa_decode_combine(const float* part_o, const float* part_ml, int nsplit,
                                                         void* out, int out_bf16) {
    constexpr int MAXS = 256;
    __shared__ float s_w[MAXS];
    __shared__ float s_inv;
    const int64_t bh = blockIdx.x;
    const int d = threadIdx.x;
    const float* ml = part_ml + bh * nsplit * 2;
    if (d < 64) {
        float mm = -__builtin_huge_valf();
        for (int sp = d; sp < nsplit; sp += 64) mm = fmaxf(mm, ml[2 * sp]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) mm = fmaxf(mm, __shfl_xor(mm, o, 64));
        float ll = 0.0f;
        for (int sp = d; sp < nsplit; sp += 64) {
            const float ms = ml[2 * sp];
            const float w = (ms == -__builtin_huge_valf()) ? 0.0f : __builtin_amdgcn_exp2f(ms - mm);
            s_w[sp] = w;
            ll = fmaf(ml[2 * sp + 1], w, ll);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) ll += __shfl_xor(ll, o, 64);
        if (d == 0) s_inv = ll > 0.0f ? 1.0f / ll : 0.0f;
    }
    __syncthreads();
    const float* po = part_o + bh * nsplit * D + d;
    float o0 = 0.0f, o1 = 0.0f, o2 = 0.0f, o3 = 0.0f;
    int sp = 0;
    for (; sp + 4 <= nsplit; sp += 4) {
        o0 = fmaf(po[(sp + 0) * D], s_w[sp + 0], o0);
        o1 = fmaf(po[(sp + 1) * D], s_w[sp + 1], o1);
        o2 = fmaf(po[(sp + 2) * D], s_w[sp + 2], o2);
        o3 = fmaf(po[(sp + 3) * D], s_w[sp + 3], o3);
    }
    for (; sp < nsplit; ++sp) o0 = fmaf(po[sp * D], s_w[sp], o0);
    const float res = ((o0 + o1) + (o2 + o3)) * s_inv;
    if (out_bf16) reinterpret_cast<uint16_t*>(out)[bh * D + d] = f32_to_bf16_rne(res);
    else reinterpret_cast<float*>(out)[bh * D + d] = res;
}

int decode_splits(int B, int Hq, int Hkv, int S, int D, int qmode) {
    const DecGeom gm = dec_geom(D, qmode == QM_UINT4_TH, Hq / Hkv);
    const int pairs = B * Hkv;
    int splits = (1024 + pairs - 1) / pairs;                          // ~4 workgroups per CU
    const int max_useful = (S + gm.stepm - 1) / gm.stepm;             // at least one step each
    if (splits > max_useful) splits = max_useful;
    // every split, rounded up to whole steps, must fit the LDS row buffer:
    // ceil(S / splits) <= rows_max suffices because rows_max holds whole steps
    const int need = (S + gm.rows_max - 1) / gm.rows_max;
    if (splits < need) splits = need;
    if (splits < 1) splits = 1;
    return splits;
}

template <int D, bool U4, int G, bool QBF16>
static hipError_t launch_split(const DecodeArgs& a, int nsplit, bool has_mask, hipStream_t s) {
    (void)has_mask;
    const dim3 grid(nsplit, a.Hkv, a.B);
    hipLaunchKernelGGL((sdpa_decode_split<D, U4, G, QBF16>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int D, bool U4, bool QBF16>
static hipError_t dispatch_g(const DecodeArgs& a, int G, int nsplit, bool has_mask, hipStream_t s) {
    switch (G) {
    case 1: return launch_split<D, U4, 1, QBF16>(a, nsplit, has_mask, s);
    case 2: return launch_split<D, U4, 2, QBF16>(a, nsplit, has_mask, s);
    case 4: return launch_split<D, U4, 4, QBF16>(a, nsplit, has_mask, s);
    case 8: return launch_split<D, U4, 8, QBF16>(a, nsplit, has_mask, s);
    default: return hipErrorInvalidValue;
    }
}

template <int D, bool U4>
static hipError_t dispatch_q(const DecodeArgs& a, bool qbf16, int G, int nsplit, bool has_mask, hipStream_t s) {
    return qbf16 ? dispatch_g<D, U4, true>(a, G, nsplit, has_mask, s)
                 : dispatch_g<D, U4, false>(a, G, nsplit, has_mask, s);
}

hipError_t launch_sdpa_decode(const DecodeLaunch& L, hipStream_t s) {
    DecodeArgs a{L.q, L.B, L.Hq, L.Hkv, L.S, L.kc, L.ks, L.kz, L.vc, L.vs, L.vz, L.kv_len,
                 L.mask, L.mask_sb, L.sm_scale * 1.4426950408889634f, L.part_o, L.part_ml, L.err};
    const int G = L.Hq / L.Hkv;
    const bool u4 = L.qmode == QM_UINT4_TH;
    const bool has_mask = L.mask != nullptr;
    hipError_t e;
    switch (L.D) {
    case 64: e = u4 ? dispatch_q<64, true>(a, L.q_bf16, G, L.nsplit, has_mask, s)
                    : dispatch_q<64, false>(a, L.q_bf16, G, L.nsplit, has_mask, s); break;
    case 128: e = u4 ? dispatch_q<128, true>(a, L.q_bf16, G, L.nsplit, has_mask, s)
                     : dispatch_q<128, false>(a, L.q_bf16, G, L.nsplit, has_mask, s); break;
    case 256: e = u4 ? dispatch_q<256, true>(a, L.q_bf16, G, L.nsplit, has_mask, s)
                     : dispatch_q<256, false>(a, L.q_bf16, G, L.nsplit, has_mask, s); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    const unsigned nbh = (unsigned)(L.B * L.Hq);
    const int ob = L.out_bf16 ? 1 : 0;
    switch (L.D) {
    case 64: hipLaunchKernelGGL((sdpa_decode_combine<64>), dim3(nbh), dim3(64), 0, s, L.part_o, L.part_ml, L.nsplit, L.out, ob); break;
    case 128: hipLaunchKernelGGL((sdpa_decode_combine<128>), dim3(nbh), dim3(128), 0, s, L.part_o, L.part_ml, L.nsplit, L.out, ob); break;
    default: hipLaunchKernelGGL((sdpa_decode_combine<256>), dim3(nbh), dim3(256), 0, s, L.part_o, L.part_ml, L.nsplit, L.out, ob); break;
    }
    return hipGetLastError();
}

}  // namespace kvq
