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

template <int D, bool U4, int G, bool QBF16>
__global__ __launch_bounds__(256) void sdpa_decode_split(DecodeArgs a) {
    constexpr int NB = G * (U4 ? 32 : 16) >= 128 ? 2 : 4;    // steps per softmax block
    constexpr int ROWB = U4 ? D / 2 : D;
    constexpr int C = ROWB / 16;          // lanes per row
    constexpr int R = 64 / C;             // rows per wave step
    constexpr int E = U4 ? 32 : 16;       // elements per lane
    constexpr int NP = E / 2;             // fp16 pairs per lane
    constexpr int NL = QBF16 ? 1 : 2;     // fp16 limbs of q
    constexpr float VOFF = U4 ? 0.0f : 128.0f;      // fp32 value = code + VOFF
    constexpr int NV = G * E;                        // accumulators per lane
    constexpr int NVR = NV / R;                      // after the row-group reduce-scatter
    static_assert(C >= 2 && C <= 16 && (64 % C) == 0, "row must split over 2..16 lanes");

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = lane % C;
    const int r = lane / C;
    const int split = blockIdx.x;
    const int nsplit = gridDim.x;
    const int g = blockIdx.y;
    const int b = blockIdx.z;

    // ---- kv_len and this workgroup's slice --------------------------------
    int kv_len = a.kv_len ? *a.kv_len : a.S;
    if (kv_len < 1 || kv_len > a.S) {
        if (a.err && split == 0 && g == 0 && b == 0 && threadIdx.x == 0) atomicOr(a.err, KVQ_DEV_FLAG_KVLEN);
        kv_len = kv_len < 1 ? 1 : a.S;
    }
    constexpr int STEP = R * DEC_WAVES;
    int chunk = (kv_len + nsplit - 1) / nsplit;
    chunk = (chunk + STEP - 1) / STEP * STEP;
    const int j0 = split * chunk;
    const int j1 = min(j0 + chunk, kv_len);

    // ---- q: this lane's E elements of each of the G heads, fp16 -----------
    // One power of two for the G heads brings max|q| into [2^14, 2^15).
    uint32_t qh[G][NL][NP];
    float csc;        // sm_scale * log2(e) * 2^-k
    {
        float qv[G][E];
        float mx = 0.0f;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const int64_t off = ((int64_t)b * a.Hq + g * G + hh) * D + c * E;
#pragma unroll
            for (int i = 0; i < E; i += 8) load8<QBF16>(a.q, off + i, &qv[hh][i]);
#pragma unroll
            for (int i = 0; i < E; ++i) mx = fmaxf(mx, fabsf(qv[hh][i]));
        }
#pragma unroll
        for (int o = 1; o < C; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        int k = 0;
        if (mx > 0.0f) {
            int e;
            frexpf(mx, &e);
            k = 15 - e;
        }
        csc = ldexpf(a.sm_scale_log2, -k);
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                const float x0 = ldexpf(qv[hh][2 * i], k), x1 = ldexpf(qv[hh][2 * i + 1], k);
                const _Float16 h0v = (_Float16)x0, h1v = (_Float16)x1;
                half2_t hv = {h0v, h1v};
                qh[hh][0][i] = __builtin_bit_cast(uint32_t, hv);
                if constexpr (NL == 2) {
                    const _Float16 l0 = (_Float16)(x0 - (float)h0v), l1 = (_Float16)(x1 - (float)h1v);
                    half2_t lv = {l0, l1};
                    qh[hh][1][i] = __builtin_bit_cast(uint32_t, lv);
                }
            }
    }

    // ---- streaming loop ----------------------------------------------------
    // Blocks of NB steps: all K and V loads of a block are issued together,
    // pass A turns the K rows into scores, the running max moves once per
    // block (one unconditional rescale), pass B accumulates p * v.
    float acc[NV];
    float m[G], l[G], corr[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        m[hh] = -__builtin_huge_valf();
        l[hh] = 0.0f;
        corr[hh] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = 0.0f;

    // Uniform bases (scalar registers) + 32-bit per-lane byte offsets.
    const int64_t plane = ((int64_t)b * a.Hkv + g) * a.S;
    const uint8_t* kbase = a.kc + plane * ROWB;
    const uint8_t* vbase = a.vc + plane * ROWB;
    const uint8_t* ksb = reinterpret_cast<const uint8_t*>(a.ks + plane);
    const uint8_t* vsb = reinterpret_cast<const uint8_t*>(a.vs + plane);
    const uint8_t* kzb = reinterpret_cast<const uint8_t*>(a.kz + plane);
    const uint8_t* vzb = reinterpret_cast<const uint8_t*>(a.vz + plane);
    const bool has_mask = a.mask != nullptr;
    const uint8_t* mrow = reinterpret_cast<const uint8_t*>(a.mask + (has_mask ? (int64_t)b * a.mask_sb : 0));
    constexpr float NEG_INF = -__builtin_huge_valf();

    for (int jb0 = j0 + wave * R; jb0 < j1; jb0 += NB * STEP) {
        uint4 kq[NB], vq[NB];
        float skq[NB], svq[NB], mq[NB];
        int zkq[NB], zvq[NB];
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            const int j = jb0 + t * STEP + r;
            const uint32_t jc = (uint32_t)min(j, j1 - 1);           // a filled row
            const uint32_t off = jc * ROWB + (uint32_t)c * 16;
            kq[t] = *reinterpret_cast<const uint4*>(kbase + off);
            vq[t] = *reinterpret_cast<const uint4*>(vbase + off);
            skq[t] = *reinterpret_cast<const float*>(ksb + jc * 4);
            svq[t] = *reinterpret_cast<const float*>(vsb + jc * 4);
            zkq[t] = *reinterpret_cast<const int8_t*>(kzb + jc);
            zvq[t] = *reinterpret_cast<const int8_t*>(vzb + jc);
            const float madd = has_mask ? *reinterpret_cast<const float*>(mrow + jc * 4) * 1.4426950408889634f : 0.0f;
            mq[t] = j < j1 ? madd : NEG_INF;                        // rows past the slice never count
        }

        // pass A: scores (log2 domain) and the block max per head
        float sc[NB][G];
        float mb[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) mb[hh] = NEG_INF;
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            uint32_t kh[NP];
            codes_to_h2<U4>(kq[t], zoff_pair(zkq[t], U4), kh);
            const float ks = skq[t] * csc;
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                float d = 0.0f;
#pragma unroll
                for (int i = 0; i < NP; ++i) {
                    d = __builtin_amdgcn_fdot2(as_h2(qh[hh][0][i]), as_h2(kh[i]), d, false);
                    if constexpr (NL == 2) d = __builtin_amdgcn_fdot2(as_h2(qh[hh][1][i]), as_h2(kh[i]), d, false);
                }
                d = group_sum<C>(d);
                sc[t][hh] = fmaf(d, ks, mq[t]);
                mb[hh] = fmaxf(mb[hh], sc[t][hh]);
            }
        }

        // move the running max once per block
        float msafe[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const float mn = fmaxf(m[hh], mb[hh]);
            msafe[hh] = mn == NEG_INF ? 0.0f : mn;
            const float al = __builtin_amdgcn_exp2f(m[hh] - msafe[hh]);
            m[hh] = mn;
            l[hh] *= al;
            corr[hh] *= al;
#pragma unroll
            for (int i = 0; i < E; ++i) acc[hh * E + i] *= al;
        }

        // pass B: p * v
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            float vf[E];
            codes_to_f32<U4>(vq[t], vf);
            const float zvo = (float)zvq[t] + VOFF;
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                const float p = __builtin_amdgcn_exp2f(sc[t][hh] - msafe[hh]);
                const float pv = p * svq[t];
                l[hh] += p;
                corr[hh] = fmaf(pv, zvo, corr[hh]);
#pragma unroll
                for (int i = 0; i < E; ++i) acc[hh * E + i] = fmaf(pv, vf[i], acc[hh * E + i]);
            }
        }
    }

    // ---- merge the R row groups of the wave --------------------------------
    // Common max per head, rescale, then reduce-scatter the NV accumulators:
    // lane (r, c) ends with values [r*NVR, (r+1)*NVR) of its column chunk c.
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        float mw = m[hh];
#pragma unroll
        for (int o = C; o < 64; o <<= 1) mw = fmaxf(mw, __shfl_xor(mw, o, 64));
        const float al = (m[hh] == -__builtin_huge_valf()) ? 0.0f : __builtin_amdgcn_exp2f(m[hh] - mw);
        float lh = l[hh] * al, ch = corr[hh] * al;
#pragma unroll
        for (int o = C; o < 64; o <<= 1) {
            lh += __shfl_xor(lh, o, 64);
            ch += __shfl_xor(ch, o, 64);
        }
#pragma unroll
        for (int i = 0; i < E; ++i) acc[hh * E + i] *= al;
        m[hh] = mw;
        l[hh] = lh;
        corr[hh] = ch;
    }
    reduce_scatter<NV, 32, C>(acc, lane);

    // ---- merge the waves through LDS and write the partial -----------------
    __shared__ float s_o[DEC_WAVES][G][D];
    __shared__ float s_m[DEC_WAVES][G], s_l[DEC_WAVES][G];
#pragma unroll
    for (int i = 0; i < NVR; ++i) {
        const int v = r * NVR + i;                 // value index: head v / E, element v % E
        const int hh = v / E;
        s_o[wave][hh][c * E + v % E] = acc[i] - corr[hh];
    }
    if (lane == 0) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) { s_m[wave][hh] = m[hh]; s_l[wave][hh] = l[hh]; }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
        const int hh = idx / D, d = idx % D;
        float mm = -__builtin_huge_valf();
#pragma unroll
        for (int w = 0; w < DEC_WAVES; ++w) mm = fmaxf(mm, s_m[w][hh]);
        float o = 0.0f, ll = 0.0f;
#pragma unroll
        for (int w = 0; w < DEC_WAVES; ++w) {
            const float al = (s_m[w][hh] == -__builtin_huge_valf()) ? 0.0f : __builtin_amdgcn_exp2f(s_m[w][hh] - mm);
            o = fmaf(s_o[w][hh][d], al, o);
            ll = fmaf(s_l[w][hh], al, ll);
        }
        const int64_t ph = ((int64_t)b * a.Hq + g * G + hh) * nsplit + split;
        a.part_o[ph * D + d] = o;
        if (d == 0) {
            a.part_ml[ph * 2] = mm;
            a.part_ml[ph * 2 + 1] = ll;
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

int decode_splits(int B, int Hkv, int S, int D, int qmode) {
    const int rowb = qmode == QM_UINT4_TH ? D / 2 : D;
    const int rows_per_step = (64 / (rowb / 16)) * DEC_WAVES;
    const int pairs = B * Hkv;
    int splits = (1024 + pairs - 1) / pairs;                        // ~4 workgroups per CU
    if (splits > 256) splits = 256;                                  // combine stages <= 256 (m, l)
    const int max_useful = (S + rows_per_step - 1) / rows_per_step;  // at least one step each
    if (splits > max_useful) splits = max_useful;
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
