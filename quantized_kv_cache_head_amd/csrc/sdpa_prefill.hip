// sdpa_prefill.hip -- chunked-prefill attention on MFMA over a quantized cache.
//
// What is computed (pytorch/executorch PR 20351, commit notes): the Lq query
// rows of a chunk sit at positions [kv_len - Lq, kv_len); row r attends keys
// j < kv_len, and with mask_is_causal only j <= kv_len - Lq + r.  The KV loop
// of a tile of rows stops at loop_end = min(kv_len, kv_len - Lq + max_row + 1)
// (the per-tile causal upper bound); skipped tiles would be fully masked, so
// the result is bit-identical to scanning every tile below kv_len.  GQA and
// the softmax scale follow abaddon's KvCache::forward_attention; an optional
// additive 0 / -inf mask is PR 24473's ring/sink mask.
//
// Mapping on gfx950 (256 threads = 4 waves, one workgroup per (b, kv head,
// tile of query rows), all G query heads of the KV head in the same
// workgroup so each K/V tile is dequantized once for all of them):
//  * Per 64-key tile the workgroup dequantizes K and V into LDS as fp16
//    holding the exact integers (code - zp) (|.| <= 255), K row-major
//    [key][d], V transposed [d][key]; the per-key scales are folded into the
//    softmax (K) and into P (V), so dequantization adds no rounding.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_f16: keys are the MFMA rows, so each
//    lane holds 16 keys of one query column and the softmax max/sum need only
//    one exchange between the two 32-lane halves.
//  * P^T leaves the MFMA accumulator in the layout the next MFMA takes as its B
//    operand; the V^T tile in LDS is stored in the matching key order, so
//    O^T += V^T P^T needs no shuffles.  Each A operand read from LDS feeds QB
//    MFMAs (QB query blocks of 32 per wave).
//  * q is rescaled by a power of two so fp16 holds it (exact for bf16 input);
//    fp32 input uses hi + lo fp16 limbs for Q.  P * scale_v enters the PV
//    MFMA as hi + lo fp16 limbs.
//  * Online softmax in the log2 domain with lazy rescaling (only when a
//    query's max grows by more than 8).
//  * Workgroups of one KV head are placed on the same XCD so its K/V stream
//    is shared through that XCD's L2.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

struct PrefillArgs {
    const void* q;
    int B, Hq, Hkv, S, Lq, n_qtiles;
    const uint8_t* kc;
    const float* ks;
    const int8_t* kz;
    const uint8_t* vc;
    const float* vs;
    const int8_t* vz;
    const int32_t* kv_len;
    const float* mask;
    int causal, no_skip, out_bf16;
    float sm_scale_log2;
    void* out;
    int32_t* err;
};

constexpr int PF_BN = 64;        // keys per tile
constexpr float PF_TAU = 8.0f;   // lazy rescale threshold (log2 units)

// Position of key k32 (0..31) of a 32-key block in the V^T LDS row: the order
// in which the S^T accumulator hands keys to the PV MFMA (half h, sub-block s,
// element e of key (2s + e/4) * 8 + h * 4 + e % 4 go to h * 16 + s * 8 + e).
__device__ __forceinline__ int vt_pos32(int k32) {
    return (((k32 >> 2) & 1) << 4) | (((k32 >> 4) & 1) << 3) | (((k32 >> 3) & 1) << 2) | (k32 & 3);
}

__device__ __forceinline__ uint32_t h2_sub(uint32_t a, uint32_t b) {
    half2_t r = __builtin_bit_cast(half2_t, a) - __builtin_bit_cast(half2_t, b);
    return __builtin_bit_cast(uint32_t, r);
}

// 4 code bytes -> 4 (int8) or 8 (4-bit) exact fp16 values (code - zp), as
// pairs of consecutive elements.  off = fp16 pair holding (OFFSET + zp) twice.
template <bool U4>
__device__ __forceinline__ void dq_dword(uint32_t w, uint32_t off, uint32_t* out) {
    if constexpr (!U4) {
        const uint32_t u = w ^ 0x80808080u;
        out[0] = h2_sub(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u), off);
        out[1] = h2_sub(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u), off);
    } else {
        const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
        out[0] = h2_sub(__builtin_amdgcn_perm(hi, lo, 0x0C040C00u) | 0x64006400u, off);
        out[1] = h2_sub(__builtin_amdgcn_perm(hi, lo, 0x0C050C01u) | 0x64006400u, off);
        out[2] = h2_sub(__builtin_amdgcn_perm(hi, lo, 0x0C060C02u) | 0x64006400u, off);
        out[3] = h2_sub(__builtin_amdgcn_perm(hi, lo, 0x0C070C03u) | 0x64006400u, off);
    }
}

// 4-bit codes with fewer operations: 8 codes (one dword, element 2i in the
// low nibble of byte i) -> 4 fp16 pairs (code - zp) in the order
// (e0,e2) (e4,e6) (e1,e3) (e5,e7): the low and the high nibbles are each
// placed under the fp16 exponent of 1024 by one byte permute with a 0x64
// constant word.  Element order within each group of 8 is therefore
// U4_ORDER[p] for position p; q takes the same order for q . k, and the V^T
// transpose undoes it.
__device__ constexpr int U4_ORDER[8] = {0, 2, 4, 6, 1, 3, 5, 7};
__device__ __forceinline__ void dq_dword_u4p(uint32_t w, uint32_t off, uint32_t* out) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    out[0] = h2_sub(__builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u), off);
    out[1] = h2_sub(__builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u), off);
    out[2] = h2_sub(__builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u), off);
    out[3] = h2_sub(__builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u), off);
}

__device__ __forceinline__ uint32_t zp_pair(int zp, bool u4) {
    // fp16 of (1024 + 128 + zp) for int8 (codes enter as 1024 + (c + 128)),
    // (1024 + zp) for 4-bit; exact integers below 2048.
    const _Float16 h = (_Float16)(float)((u4 ? 1024 : 1152) + zp);
    half2_t v = {h, h};
    return __builtin_bit_cast(uint32_t, v);
}

template <int D, bool U4, int QB, int QL, int PL>
__global__ __launch_bounds__(256, 1) void sdpa_prefill_mfma(PrefillArgs a) {
    constexpr int ROWB = U4 ? D / 2 : D;
    constexpr int KPITCH = D + 8;          // fp16 elements per K row in LDS
    constexpr int VPITCH = PF_BN + 8;      // fp16 elements per V^T row in LDS
    constexpr int NKB = D / 16;            // MFMA k-steps for q.k
    constexpr int NDB = D / 32;            // d blocks of the output

    __shared__ __attribute__((aligned(16))) _Float16 k_lds[PF_BN * KPITCH];
    __shared__ __attribute__((aligned(16))) _Float16 v_lds[D * VPITCH];
    __shared__ float c_lds[PF_BN];         // key scale * softmax scale (0 past kv_len)
    __shared__ float sv_lds[PF_BN];        // value scale (0 past kv_len)
    // raw code tiles (K rows then V rows), double-buffered: the next tile's
    // bytes stream in with global_load_lds while this tile is computed
    constexpr int RAWB = 2 * PF_BN * ROWB;
    __shared__ __attribute__((aligned(16))) uint8_t raw_lds[2][RAWB];
    // per-key metadata of a tile, double-buffered: (k scale, v scale, k zp, v zp)
    __shared__ float mks_lds[2][PF_BN], mvs_lds[2][PF_BN];
    __shared__ int mkz_lds[2][PF_BN], mvz_lds[2][PF_BN];
    __shared__ float red_lds[4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hl = lane >> 5;              // 32-lane half
    const int l32 = lane & 31;
    const int G = a.Hq / a.Hkv;
    const int QT = 128 * QB / G;           // query rows of each head in this tile
    const bool has_mask = a.mask != nullptr;

    // ---- workgroup -> (b, kv head, query tile), XCD-aware ------------------
    int L = blockIdx.x;
    const int NB = gridDim.x;
    if ((NB & 7) == 0) L = (blockIdx.x & 7) * (NB >> 3) + (blockIdx.x >> 3);
    const int qtile = L % a.n_qtiles;
    const int bg = L / a.n_qtiles;
    const int g = bg % a.Hkv;
    const int b = bg / a.Hkv;
    const int r0 = qtile * QT;

    int kv_len = a.kv_len ? *a.kv_len : a.S;
    if (kv_len < a.Lq || kv_len > a.S) {
        if (a.err && blockIdx.x == 0 && tid == 0) atomicOr(a.err, KVQ_DEV_FLAG_KVLEN);
        kv_len = kv_len < a.Lq ? a.Lq : a.S;
    }
    const int row_last = min(r0 + QT, a.Lq) - 1;
    const int qpos0 = kv_len - a.Lq;       // absolute position of query row 0
    int loop_end = kv_len;
    if (a.causal && !a.no_skip) loop_end = min(kv_len, qpos0 + row_last + 1);

    // ---- this lane's query columns ------------------------------------------
    int q_head[QB], q_row[QB];
    bool q_live[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qr = (wave * QB + qb) * 32 + l32;   // index in (head, row) of the tile
        q_head[qb] = g * G + qr / QT;
        q_row[qb] = r0 + qr % QT;
        q_live[qb] = q_row[qb] < a.Lq;
    }

    // ---- Q^T operands: fp16, prescaled by 2^k (k shared by the workgroup) ----
    // pass 1: max |q| over the workgroup; pass 2: reload and convert.
    float qmax = 0.0f;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        if (!q_live[qb]) continue;
        const int64_t qoff = (((int64_t)b * a.Hq + q_head[qb]) * a.Lq + q_row[qb]) * D;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            float v[8];
            load8<QL == 1>(a.q, qoff + hl * (D / 2) + kb * 8, v);
#pragma unroll
            for (int e = 0; e < 8; ++e) qmax = fmaxf(qmax, fabsf(v[e]));
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, o, 64));
    if (lane == 0) red_lds[wave] = qmax;
    __syncthreads();
    qmax = fmaxf(fmaxf(red_lds[0], red_lds[1]), fmaxf(red_lds[2], red_lds[3]));
    int qk = 0;
    if (qmax > 0.0f) {
        int e;
        frexpf(qmax, &e);
        qk = 15 - e;
    }
    const float rs = ldexpf(a.sm_scale_log2, -qk);
    half8_t qh[QB][NKB][QL];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int64_t qoff = (((int64_t)b * a.Hq + q_head[qb]) * a.Lq + (q_live[qb] ? q_row[qb] : 0)) * D;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            float v[8];
            load8<QL == 1>(a.q, qoff + hl * (D / 2) + kb * 8, v);
            half8_t hi, lo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = q_live[qb] ? ldexpf(v[U4 ? U4_ORDER[e] : e], qk) : 0.0f;
                hi[e] = (_Float16)x;
                lo[e] = (_Float16)(x - (float)hi[e]);
            }
            qh[qb][kb][0] = hi;
            if constexpr (QL == 2) qh[qb][kb][QL - 1] = lo;
        }
    }

    // ---- state ---------------------------------------------------------------
    float16_t o_acc[NDB][QB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int i = 0; i < 16; ++i) o_acc[db][qb][i] = 0.0f;
    float m_run[QB], l_run[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) { m_run[qb] = -__builtin_huge_valf(); l_run[qb] = 0.0f; }

    const int64_t plane = ((int64_t)b * a.Hkv + g) * a.S;
    const uint8_t* kcodes = a.kc + plane * ROWB;
    const uint8_t* vcodes = a.vc + plane * ROWB;
    const int n_tiles = (loop_end + PF_BN - 1) / PF_BN;
    const int diag_lo = qpos0 + r0;        // keys <= this are visible to every row of the tile

    // Asynchronous copy of tile tt's K and V code rows into raw_lds[buf]: a
    // workgroup-wide step moves 256 x 16 bytes; lane l of wave w in step i
    // fills bytes i*4096 + w*1024 + l*16 of the tile (rows past the cache end
    // read the last row: they are masked).
    constexpr int TILEB = PF_BN * ROWB;                // bytes of a K (or V) tile
    constexpr int RSTEPS = (TILEB + 4095) / 4096;     // steps per K (or V) tile
    static_assert(TILEB % 4096 == 0 || TILEB < 4096, "raw tile steps");
    auto fetch_raw = [&](int tt, int buf) {
        const int jt = tt * PF_BN;
#pragma unroll
        for (int i = 0; i < RSTEPS; ++i) {
            const int off = i * 4096 + tid * 16;
            if (TILEB < 4096 && off >= TILEB) continue;   // whole waves past a small tile

            const int key = off / ROWB, col = off % ROWB;
            const int64_t j = min(jt + key, a.S - 1);
            __attribute__((address_space(3))) void* lk =
                (__attribute__((address_space(3))) void*)(raw_lds[buf] + i * 4096 + wave * 1024);
            __attribute__((address_space(3))) void* lv =
                (__attribute__((address_space(3))) void*)(raw_lds[buf] + PF_BN * ROWB + i * 4096 + wave * 1024);
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(kcodes + j * ROWB + col),
                                             lk, 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(vcodes + j * ROWB + col),
                                             lv, 16, 0, 0);
        }
    };
    // per-key metadata of tile tt: loaded into registers (threads < 64), stored
    // to the metadata buffer later, when the loads have landed
    float mk_s = 0.0f, mv_s = 0.0f;
    int mk_z = 0, mv_z = 0;
    auto fetch_meta = [&](int tt) {
        if (tid < PF_BN) {
            const int j = min(tt * PF_BN + tid, a.S - 1);
            mk_s = a.ks[plane + j];
            mv_s = a.vs[plane + j];
            mk_z = a.kz[plane + j];
            mv_z = a.vz[plane + j];
        }
    };
    auto store_meta = [&](int buf) {
        if (tid < PF_BN) {
            mks_lds[buf][tid] = mk_s;
            mvs_lds[buf][tid] = mv_s;
            mkz_lds[buf][tid] = mk_z;
            mvz_lds[buf][tid] = mv_z;
        }
    };
    if (n_tiles > 0) {
        fetch_meta(0);
        fetch_raw(0, 0);
        store_meta(0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    for (int t = 0; t < n_tiles; ++t) {
        const int j0 = t * PF_BN;
        const int cur = t & 1;
        // the next tile's metadata, then its code rows, go out first (the
        // metadata is waited for below without waiting for the code rows)
        if (t + 1 < n_tiles) {
            fetch_meta(t + 1);
            fetch_raw(t + 1, cur ^ 1);
        }
        const uint8_t* rk = raw_lds[cur];
        const uint8_t* rv = raw_lds[cur] + PF_BN * ROWB;
        // ---------------- stage: dequantize K and V^T into LDS ----------------
        {
            constexpr int CPR = ROWB / 16;                 // 16-byte chunks per K row
            constexpr int NCH = PF_BN * CPR;
#pragma unroll
            for (int c = tid; c < NCH; c += 256) {
                const int kk = c / CPR, ch = c % CPR;
                const uint4 w = *reinterpret_cast<const uint4*>(rk + kk * ROWB + ch * 16);
                const uint32_t off = zp_pair(mkz_lds[cur][kk], U4);
                uint32_t hv[U4 ? 16 : 8];
                if constexpr (U4) {
                    dq_dword_u4p(w.x, off, hv + 0);
                    dq_dword_u4p(w.y, off, hv + 4);
                    dq_dword_u4p(w.z, off, hv + 8);
                    dq_dword_u4p(w.w, off, hv + 12);
                } else {
                    dq_dword<false>(w.x, off, hv + 0);
                    dq_dword<false>(w.y, off, hv + 2);
                    dq_dword<false>(w.z, off, hv + 4);
                    dq_dword<false>(w.w, off, hv + 6);
                }
                uint4* dst = reinterpret_cast<uint4*>(k_lds + kk * KPITCH + ch * (U4 ? 32 : 16));
#pragma unroll
                for (int i = 0; i < (U4 ? 4 : 2); ++i) dst[i] = make_uint4(hv[4 * i], hv[4 * i + 1], hv[4 * i + 2], hv[4 * i + 3]);
            }
            // V^T: unit = 8 keys (one LDS run) x 8 d
            constexpr int NDG = D / 8;
            for (int u = tid; u < 8 * NDG; u += 256) {
                const int dg = u % NDG, kg = u / NDG;       // kg = kbk*4 + h*2 + s
                const int kbk = kg >> 2, hh = (kg >> 1) & 1, s = kg & 1;
                uint32_t pr[8][4];                          // per key: 4 fp16 pairs
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int k64 = kbk * 32 + (2 * s + (e >> 2)) * 8 + hh * 4 + (e & 3);
                    const uint32_t off = zp_pair(mvz_lds[cur][k64], U4);
                    const uint8_t* src = rv + k64 * ROWB + (U4 ? dg * 4 : dg * 8);
                    if constexpr (U4) {
                        dq_dword_u4p(*reinterpret_cast<const uint32_t*>(src), off, pr[e]);
                    } else {
                        const uint2 w2 = *reinterpret_cast<const uint2*>(src);
                        dq_dword<false>(w2.x, off, pr[e]);
                        dq_dword<false>(w2.y, off, pr[e] + 2);
                    }
                }
                // 16-byte chunk of the V^T row, XOR-swizzled by the row's group of
                // 8 so that the 32 lanes of a store (rows 8 apart) spread over the
                // banks; the PV operand read applies the same swizzle
                const int chunk = (kbk * 32 + hh * 16 + s * 8) / 8;
#pragma unroll
                for (int dd = 0; dd < 8; ++dd) {
                    // gather element dd of each of the 8 keys: int8 pairs hold
                    // (dd, dd+1); 4-bit pairs hold the U4_ORDER arrangement
                    const int pq = U4 ? ((dd & 1) * 2 + (dd >> 2)) : (dd >> 1);
                    const int ph = U4 ? ((dd >> 1) & 1) : (dd & 1);
                    const uint32_t sel = ph ? 0x07060302u : 0x05040100u;
                    uint32_t o4[4];
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2)
                        o4[e2] = __builtin_amdgcn_perm(pr[2 * e2 + 1][pq], pr[2 * e2][pq], sel);
                    *reinterpret_cast<uint4*>(v_lds + (dg * 8 + dd) * VPITCH + (chunk ^ (dg & 7)) * 8) =
                        make_uint4(o4[0], o4[1], o4[2], o4[3]);
                }
            }
            if (tid < PF_BN) {
                const int j = j0 + tid;
                const bool in = j < kv_len;
                c_lds[tid] = in ? mks_lds[cur][tid] * rs : 0.0f;
                sv_lds[tid] = in ? mvs_lds[cur][tid] : 0.0f;
            }
            if (t + 1 < n_tiles) store_meta(cur ^ 1);
        }
        __syncthreads();

        // Each 32-key block: S^T = K Q^T, softmax, O^T += V^T P^T.
        const bool tile_mask = (a.causal && j0 + PF_BN - 1 > diag_lo) || (j0 + PF_BN > kv_len) || has_mask;
#pragma unroll
        for (int kbk = 0; kbk < 2; ++kbk) {
            float16_t st[QB];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int i = 0; i < 16; ++i) st[qb][i] = 0.0f;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const half8_t av = *reinterpret_cast<const half8_t*>(
                    k_lds + (kbk * 32 + l32) * KPITCH + hl * (D / 2) + kb * 8);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                    for (int ql = 0; ql < QL; ++ql)
                        st[qb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, qh[qb][kb][ql], st[qb], 0, 0, 0);
            }

            // softmax: lane holds keys j0 + kbk*32 + (i/4)*8 + hl*4 + i%4
            half8_t pb[2][QB][PL];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                float tmax = -__builtin_huge_valf();
                const int lim = a.causal ? qpos0 + q_row[qb] : kv_len - 1;   // last visible key
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const float4 c4 = *reinterpret_cast<const float4*>(c_lds + kbk * 32 + i4 * 8 + hl * 4);
                    const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) {
                        const int i = i4 * 4 + ii;
                        float v = st[qb][i] * cv[ii];
                        if (tile_mask) {
                            const int key = j0 + kbk * 32 + i4 * 8 + hl * 4 + ii;
                            if (has_mask && key < kv_len && q_live[qb])
                                v += a.mask[(int64_t)q_row[qb] * a.S + key] * 1.4426950408889634f;
                            if (key > lim || key >= kv_len || !q_live[qb]) v = -__builtin_huge_valf();
                        }
                        st[qb][i] = v;
                        tmax = fmaxf(tmax, v);
                    }
                }
                tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
                const bool upd = tmax > m_run[qb] + PF_TAU;
                if (__any(upd)) {
                    const float mn = upd ? tmax : m_run[qb];
                    const float al = (m_run[qb] == -__builtin_huge_valf()) ? 0.0f : __builtin_amdgcn_exp2f(m_run[qb] - mn);
                    m_run[qb] = mn;
                    l_run[qb] *= al;
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int i = 0; i < 16; ++i) o_acc[db][qb][i] *= al;
                }
                // a masked score is -inf and gives p = 2^-inf = 0; msafe keeps
                // -inf - (-inf) out of a row that has seen no key yet
                const float msafe = m_run[qb] == -__builtin_huge_valf() ? 0.0f : m_run[qb];
                float lsum = 0.0f;
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    half8_t ph, plo;
#pragma unroll
                    for (int e4 = 0; e4 < 2; ++e4) {
                        const float4 s4 = *reinterpret_cast<const float4*>(sv_lds + kbk * 32 + (sb * 2 + e4) * 8 + hl * 4);
                        const float svv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
                        for (int ii = 0; ii < 4; ii += 2) {
                            const int e = e4 * 4 + ii;
                            const float p0 = __builtin_amdgcn_exp2f(st[qb][sb * 8 + e] - msafe);
                            const float p1 = __builtin_amdgcn_exp2f(st[qb][sb * 8 + e + 1] - msafe);
                            lsum += p0 + p1;
                            const float pv0 = p0 * svv[ii], pv1 = p1 * svv[ii + 1];
                            // hi limb rounded toward zero, lo limb = the exact fp32 remainder in fp16
                            const half2_t h2 = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(pv0, pv1));
                            ph[e] = h2[0];
                            ph[e + 1] = h2[1];
                            if constexpr (PL == 2) {
                                const half2_t l2 = __builtin_bit_cast(
                                    half2_t, __builtin_amdgcn_cvt_pkrtz(pv0 - (float)h2[0], pv1 - (float)h2[1]));
                                plo[e] = l2[0];
                                plo[e + 1] = l2[1];
                            }
                        }
                    }
                    pb[sb][qb][0] = ph;
                    if constexpr (PL == 2) pb[sb][qb][PL - 1] = plo;
                }
                l_run[qb] += lsum;
            }

            // O^T += V^T P^T over these 32 keys (two MFMA k-steps of 16)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    const int vrow = db * 32 + l32;
                    const half8_t av = *reinterpret_cast<const half8_t*>(
                        v_lds + vrow * VPITCH + (((kbk * 32 + hl * 16 + sb * 8) / 8) ^ ((vrow >> 3) & 7)) * 8);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                        for (int pl = 0; pl < PL; ++pl)
                            o_acc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, pb[sb][qb][pl], o_acc[db][qb], 0, 0, 0);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0);                // the next tile's code rows have landed
        __syncthreads();
    }

    // ---- epilogue: normalize and store ---------------------------------------
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float lt = l_run[qb] + __shfl_xor(l_run[qb], 32, 64);
        if (!q_live[qb]) continue;
        const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
        const int64_t obase = (((int64_t)b * a.Hq + q_head[qb]) * a.Lq + q_row[qb]) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int d = db * 32 + i4 * 8 + hl * 4;
                const float v0 = o_acc[db][qb][i4 * 4 + 0] * inv, v1 = o_acc[db][qb][i4 * 4 + 1] * inv;
                const float v2 = o_acc[db][qb][i4 * 4 + 2] * inv, v3 = o_acc[db][qb][i4 * 4 + 3] * inv;
                if (a.out_bf16) {
                    const uint32_t w0 = (uint32_t)f32_to_bf16_rne(v0) | ((uint32_t)f32_to_bf16_rne(v1) << 16);
                    const uint32_t w1 = (uint32_t)f32_to_bf16_rne(v2) | ((uint32_t)f32_to_bf16_rne(v3) << 16);
                    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + obase + d) = make_uint2(w0, w1);
                } else {
                    *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + obase + d) = make_float4(v0, v1, v2, v3);
                }
            }
    }
}

template <int D, bool U4, int QB, int QL, int PL>
static hipError_t launch_pf(const PrefillArgs& a, hipStream_t s) {
    const int G = a.Hq / a.Hkv;
    const int QT = 128 * QB / G;
    PrefillArgs aa = a;
    aa.n_qtiles = (a.Lq + QT - 1) / QT;
    const unsigned blocks = (unsigned)(a.B * a.Hkv * aa.n_qtiles);
    hipLaunchKernelGGL((sdpa_prefill_mfma<D, U4, QB, QL, PL>), dim3(blocks), dim3(256), 0, s, aa);
    return hipGetLastError();
}

template <int D, bool U4>
static hipError_t dispatch_pf(const PrefillArgs& a, bool q_bf16, hipStream_t s) {
    // bf16 queries: one fp16 limb for Q (exact), two query blocks per wave
    // (one at D = 256, where two do not fit the register file).  fp32
    // queries: hi + lo limbs for Q, one query block per wave.  P * scale_v
    // always goes in as hi + lo fp16 limbs (about 22 bits).
    constexpr int QB = D >= 256 ? 1 : 2;
    if (q_bf16) return launch_pf<D, U4, QB, 1, 2>(a, s);
    return launch_pf<D, U4, 1, 2, 2>(a, s);
}

hipError_t launch_sdpa_prefill(const PrefillLaunch& L, hipStream_t s) {
    PrefillArgs a{L.q, L.B, L.Hq, L.Hkv, L.S, L.Lq, 0, L.kc, L.ks, L.kz, L.vc, L.vs, L.vz, L.kv_len,
                  L.mask, L.causal ? 1 : 0, L.no_skip ? 1 : 0, L.out_bf16 ? 1 : 0,
                  L.sm_scale * 1.4426950408889634f, L.out, L.err};
    const int G = L.Hq / L.Hkv;
    if (G < 1 || G > 8 || (G & (G - 1))) return hipErrorNotSupported;
    const bool u4 = L.qmode == QM_UINT4_TH;
    switch (L.D) {
    case 64: return u4 ? dispatch_pf<64, true>(a, L.q_bf16, s) : dispatch_pf<64, false>(a, L.q_bf16, s);
    case 128: return u4 ? dispatch_pf<128, true>(a, L.q_bf16, s) : dispatch_pf<128, false>(a, L.q_bf16, s);
    case 256: return u4 ? dispatch_pf<256, true>(a, L.q_bf16, s) : dispatch_pf<256, false>(a, L.q_bf16, s);
    default: return hipErrorNotSupported;
    }
}

}  // namespace kvq
