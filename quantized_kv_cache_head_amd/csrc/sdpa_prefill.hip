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
// Mapping on gfx950 (512 threads = 8 waves, one workgroup per (b, kv head,
// tile of 128 query columns), a column being one (query head, row) pair; all
// G query heads of the KV head share the workgroup, so each K/V tile is read
// and dequantized once for all of them):
//  * Each wave owns 16 query columns.  S^T = K Q^T and O^T += V^T P^T run on
//    v_mfma_f32_16x16x32_f16 with keys as the MFMA rows, so a lane holds 8
//    keys of one column and the softmax max / sum need two lane swaps.
//  * Per 32-key tile the codes become fp16 holding the exact integers
//    (code - zp) (|.| <= 255) in LDS: K row-major [key][d], V transposed
//    [d][key] in the key order in which the S^T accumulator hands P to the
//    PV MFMA.  Per-key scales fold into the softmax (K) and into P (V), so
//    dequantization adds no rounding.
//  * q is rescaled by a power of two that puts max|q| of the tile in
//    [2^14, 2^15); a bf16 element is exact in fp16 unless it lies more than
//    2^31 below that maximum (it then rounds on fp16's subnormal grid, an
//    error below 2^-39 of max|q|).  fp32 input uses hi + lo fp16 limbs.
//  * Online softmax in the log2 domain with a lazily raised reference m per
//    query column that also carries the size of the V scales: p' = 2^(s - m)
//    and P * scale_v enters the PV MFMA as hi + lo fp16 limbs of
//    p' * scale_v.  m is raised (and the column's O and l rescaled by the
//    same factor) only when a tile's bound max(s) + log2 max(scale_v) passes
//    m + 15, and then set 7.5 below that bound: p' * scale_v stays below
//    2^15 (fp16 ends at 2^16) and starts near 2^7.5, far above fp16's
//    subnormals, whether the V scales are tiny or in the thousands.  O and l
//    share the factor 2^m, which cancels in O / l.  Without a mask the scale
//    maximum is one value for the workgroup's whole key range, found by a
//    pass over its V scales before the tile loop (every slot below kv_len
//    holds a written token then), so the tile loop pays one add for it.
//    With a mask it runs per tile over the keys below kv_len that the mask
//    leaves visible to the column (a hidden slot's scale may hold anything).
//    The two choices round differently, so a zero mask and no mask agree
//    within rounding rather than to the bit.
//  * Software pipeline over tiles: the raw codes of tile t+2 stream into LDS
//    (global_load_lds) and tile t+1 is dequantized while tile t's MFMAs run;
//    one barrier per tile.  The tile loop is compiled separately for the
//    K-dequantizing and the V-dequantizing waves, so a wave's QK MFMAs and its
//    dequantization share one basic block, and the scheduler is asked to
//    issue them interleaved (one MFMA, then four VALU instructions): the
//    VALU work runs while the matrix core is busy instead of after it.
//  * Workgroups of one KV head are placed on the same XCD so its K/V stream
//    is shared through that XCD's L2.
//  * Block caches (a scale per 32 elements: FP8-E4M3, FP8-E5M2 or int8 with
//    an fp32 scale, MX-FP8 / MX-FP4 with an E8M0 scale; the IndexerQuantCache
//    operator page's formats): the codes become exact fp16 through the gfx950
//    conversions (int8: the exponent trick).  One QK k-step of 32 d is exactly one
//    scale block, so each block's partial S^T is scaled per key in fp32 and
//    summed; V^T rows stay in d order so a 16-row output block lies in one
//    scale block, and P enters that block's PV product scaled by the keys'
//    V scales of that block.  Raw rows are read below kv_len only.
#include <type_traits>
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

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
    int kv_len_sb;         // 0: one kv_len for the batch; 1: one per batch row
    const float* mask;
    int causal, no_skip, out_bf16;
    float sm_scale_log2;
    void* out;
    int32_t* err;
    int kv_splits;         // workgroups per query tile along the key range (gridDim.y)
    float* part_o;         // kv_splits > 1: [B * Hq * Lq, kv_splits, D] unnormalized outputs
    float* part_ml;        //                [B * Hq * Lq, kv_splits, 2] (max, sum) in log2 units
};

// Reference raise rule (log2 units): raised when the bound on p' * scale_v
// passes 2^PF_PV_HI, then set so that the bound is 2^PF_PV_SET; log2 of the
// V-scale bound taken as at least PF_LSV_MIN (a column with no nonzero live
// V scale adds nothing to O but still counts its p' in l).
constexpr float PF_PV_HI = 15.0f;
constexpr float PF_PV_SET = 7.5f;
constexpr float PF_LSV_MIN = -48.0f;

__device__ __forceinline__ uint32_t h2_sub(uint32_t a, uint32_t b) {
    half2_t r = __builtin_bit_cast(half2_t, a) - __builtin_bit_cast(half2_t, b);
    return __builtin_bit_cast(uint32_t, r);
}

// 4 int8 code bytes -> 4 exact fp16 values (code - zp) as 2 pairs of
// consecutive elements: (code + 128) is placed under the fp16 exponent of
// 1024 by a byte permute; off = fp16 pair holding (1152 + zp) twice.
__device__ __forceinline__ void dq_dword_i8(uint32_t w, uint32_t off, uint32_t* out) {
    const uint32_t u = w ^ 0x80808080u;
    out[0] = h2_sub(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u), off);
    out[1] = h2_sub(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u), off);
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

// Largest of p[0, n) (non-negative floats; 0 for n <= 0) over the lanes of a
// 512-thread workgroup, this lane's share: 16-byte loads where aligned.
__device__ __forceinline__ float range_max_f32(const float* p, int n, int tid) {
    const int h = min((int)(((16 - ((uintptr_t)p & 15)) & 15) >> 2), max(n, 0));
    float x = tid < h ? p[tid] : 0.0f;
    const float4* p4 = reinterpret_cast<const float4*>(p + h);
    const int n4 = (n - h) >> 2;
#pragma unroll 16
    for (int i = tid; i < n4; i += 512) {
        const float4 v = p4[i];
        x = fmaxf(x, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
    }
    const int tl = h + 4 * max(n4, 0);
    if (tid < n - tl) x = fmaxf(x, p[tl + tid]);
    return x;
}

// V scales are staged finite: a NaN or infinite one (which only a slot that
// was never written can hold, behind the mask) becomes 0, so a dropped key's
// p = 0 times its scale is exactly 0 without a select per key in the tile loop.
__device__ __forceinline__ float finite_or_0(float x) { return __builtin_fabsf(x) <= 3.402823466e38f ? x : 0.0f; }

// max of two floats that are never signalling NaNs (scores, -inf), as one
// v_max_f32: fmaxf on the result of a lane swap, which the compiler cannot
// prove quiet, would first quieten both inputs under the IEEE mode
__device__ __forceinline__ float fmax_q(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// x from another lane of the row by the DPP control CTRL (all rows, all banks)
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ uint32_t zp_pair(int zp, bool u4) {
    // fp16 of (1024 + 128 + zp) for int8 (codes enter as 1024 + (c + 128)),
    // (1024 + zp) for 4-bit; exact integers below 2048.
    const _Float16 h = (_Float16)(float)((u4 ? 1024 : 1152) + zp);
    half2_t v = {h, h};
    return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------------------
// 16 query columns per wave (v_mfma_f32_16x16x32_f16), 8 waves per workgroup
// (128 columns), tiles of 32 keys, software-pipelined:
//  * the raw code rows of tile t+2 stream into LDS (global_load_lds) while
//    tile t is processed;
//  * tile t+1 is dequantized into the second pair of fp16 tiles (waves 0-3 the
//    K rows, waves 4-7 the V^T tile) between tile t's QK MFMAs and its
//    softmax, so its VALU work runs while those MFMAs execute;
//  * one barrier per tile.
// With 16 columns the output accumulators take 64 registers at D = 256, so two
// waves share a SIMD.
// ---------------------------------------------------------------------------
constexpr int PF_BN = 32;
constexpr int PF_WAVES = 8;

// V^T column of key k (0..31) of a tile: lane group g of the PV B operand
// holds keys 4g..4g+3 of the first and of the second 16-key block (the S^T
// accumulator layout), as k-indices 8g..8g+3 and 8g+4..8g+7.
__device__ __forceinline__ int pf_col(int k) { return ((k & 15) >> 2) * 8 + (k >> 4) * 4 + (k & 3); }
// 16-byte chunk swizzles: K rows by key, V^T rows by row.  A 128-bit LDS
// read serves 16 lanes per pass; for 16 consecutive keys of a 256- or 512-byte
// K row the chunk index is XORed with 4 key bits so the 16 reads fall in
// distinct banks (measured: 3 bits left them 2-way conflicted); 128-byte rows
// (D 64) need 3.
template <int D>
__device__ __forceinline__ int pf_ksw(int key) { return D >= 128 ? (key & 15) : (key & 7); }
__device__ __forceinline__ int pf_vsw(int row) { return (row >> 1) & 3; }
// V^T rows of block caches are in natural d order (a 16-row MFMA block then
// lies inside one 32-element scale block); the stage writes 8 consecutive
// rows per thread, so the swizzle follows the row's group of 8.
__device__ __forceinline__ int pf_vswb(int row) { return (row >> 3) & 3; }

// One dword of block codes to exact fp16 pairs in element order: FP8-E4M3
// (MX-FP8 too) and FP8-E5M2, 4 per dword, and FP4-E2M1, 8 per dword (element
// 2i in the low nibble of byte i), through the gfx950 conversions at scale 1;
// int8, 4 per dword, as (code + 128) under the fp16 exponent of 1024 minus
// 1152.
template <int QM>
__device__ __forceinline__ void blk_dword(uint32_t w, uint32_t* out) {
    if constexpr (QM == QM_MXFP4E1M2_B32) {
#pragma unroll
        for (int j = 0; j < 4; ++j) out[j] = e1m2_pair_h2(w, j);
    } else if constexpr (QM == QM_MXFP4_B32) {
        out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0));
        out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1));
        out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2));
        out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3));
    } else if constexpr (QM == QM_FP8E5M2_B32) {
        out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, false));
        out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, true));
    } else if constexpr (QM == QM_INT8_B32) {
        dq_dword_i8(w, 0x64806480u, out);
    } else {
        out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
        out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
    }
}

template <int D, int QM, int QL, int PL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sdpa_prefill_mfma(PrefillArgs a) {
    constexpr bool BLK = QM >= QM_FP8E4M3_B32;      // per-32 block scales
    constexpr bool F4 = QM == QM_MXFP4_B32 || QM == QM_MXFP4E1M2_B32;  // FP4 codes, two per byte
    constexpr bool U4 = QM == QM_UINT4_TH || F4;                        // two codes per byte
    constexpr bool SC8 = F4 || QM == QM_MXFP8_B32;                      // E8M0 block scales
    constexpr bool PERM = QM == QM_UINT4_TH;         // affine 4-bit: U4_ORDER element order
    constexpr int NG = D / 32;                       // scale blocks per row (= QK k-steps)
    constexpr int BN = PF_BN;
    constexpr int ROWB = U4 ? D / 2 : D;
    constexpr int NDS = D / 32;            // QK MFMA k-steps (32 d each)
    constexpr int NDB = D / 16;            // output d-blocks (16 d each)
    constexpr int TILEB = BN * ROWB;       // raw bytes of a K (or V) tile
    constexpr int RB = ROWB / 8;           // raw bytes of one eighth of a K row
    constexpr bool KPM = RB >= 16;         // raw K tile stored part-major ([part][key])
    constexpr int DG = D / 8;              // groups of 8 d
    constexpr float NEG_INF = -__builtin_huge_valf();
    static_assert(D >= 64, "K row swizzle needs 8 chunks");

    // Every double buffer is two variables, not an array of two: the compiler
    // then sees that writes to one never alias reads of the other (and does
    // not wait for the asynchronous copies before reading the other buffer).
    __shared__ __attribute__((aligned(16))) _Float16 k_a[BN * D], k_b[BN * D];
    // V^T rows in the order R(d) = (d % 8) * DG + d / 8
    __shared__ __attribute__((aligned(16))) _Float16 v_a[D * BN], v_b[D * BN];
    __shared__ __attribute__((aligned(16))) uint8_t raw_a[2 * TILEB], raw_b[2 * TILEB];
    __shared__ __attribute__((aligned(16))) float c_a[BN], c_b[BN], s_a[BN], s_b[BN];
    __shared__ float mks_lds[2][BN], mvs_lds[2][BN];
    __shared__ int mkz_lds[2][BN], mvz_lds[2][BN];
    // block caches: block scales [group][key] as fetched (double buffer by
    // tile parity) and as used by a tile's products (double buffer by slot)
    constexpr int NBS = BLK ? NG * BN : 1;
    __shared__ float bks_lds[2][NBS], bvs_lds[2][NBS];
    __shared__ __attribute__((aligned(16))) float bk_a[NBS], bk_b[NBS], bv_a[NBS], bv_b[NBS];
    __shared__ float red_lds[PF_WAVES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lg = lane >> 4;              // lane group (0..3)
    const int l16 = lane & 15;
    const int t256 = tid & 255;            // index within the K (waves 0-3) or V (4-7) half
    const bool vhalf = tid >= 256;
    const int G = a.Hq / a.Hkv;
    const int QT = 16 * PF_WAVES / G;     // query rows of each head in this tile
    const bool has_mask = a.mask != nullptr;

    int L = blockIdx.x;
    const int NB = gridDim.x;
    if ((NB & 7) == 0) L = (blockIdx.x & 7) * (NB >> 3) + (blockIdx.x >> 3);
    const int qtile = L % a.n_qtiles;
    const int bg = L / a.n_qtiles;
    const int g = bg % a.Hkv;
    const int b = bg / a.Hkv;
    const int r0 = qtile * QT;

    int kv_len = a.kv_len ? a.kv_len[(int64_t)b * a.kv_len_sb] : a.S;
    if (kv_len < a.Lq || kv_len > a.S) {
        if (a.err && qtile == 0 && g == 0 && tid == 0) atomicOr(a.err, KVQ_DEV_FLAG_KVLEN);
        kv_len = kv_len < a.Lq ? a.Lq : a.S;
    }
    const int row_last = min(r0 + QT, a.Lq) - 1;
    const int qpos0 = kv_len - a.Lq;
    int loop_end = kv_len;
    if (a.causal && !a.no_skip) loop_end = min(kv_len, qpos0 + row_last + 1);

    // ---- this lane's query column --------------------------------------------
    const int qc = wave * 16 + l16;
    const int q_head = g * G + qc / QT;
    const int q_row = r0 + qc % QT;
    const bool q_live = q_row < a.Lq;

    // ---- Q^T operand (lane group lg holds d = ds*32 + 8*lg .. +8) ------------
    const int64_t qoff = (((int64_t)b * a.Hq + q_head) * a.Lq + (q_live ? q_row : 0)) * D;
    float qmax = 0.0f;
    if (q_live) {
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
            float v[8];
            load8<QL == 1>(a.q, qoff + ds * 32 + 8 * lg, v);
#pragma unroll
            for (int e = 0; e < 8; ++e) qmax = fmaxf(qmax, fabsf(v[e]));
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, o, 64));
    if (lane == 0) red_lds[wave] = qmax;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < PF_WAVES; ++w) qmax = fmaxf(qmax, red_lds[w]);
    int qk = 0;
    if (qmax > 0.0f) {
        int e;
        frexpf(qmax, &e);
        qk = 15 - e;
    }
    const float rs = ldexpf(a.sm_scale_log2, -qk);
    half8_t qh[NDS][QL];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
        float v[8];
        load8<QL == 1>(a.q, qoff + ds * 32 + 8 * lg, v);
        half8_t hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = q_live ? ldexpf(v[PERM ? U4_ORDER[e] : e], qk) : 0.0f;
            hi[e] = (_Float16)x;
            lo[e] = (_Float16)(x - (float)hi[e]);
        }
        qh[ds][0] = hi;
        if constexpr (QL == 2) qh[ds][QL - 1] = lo;
    }

    // ---- state ----------------------------------------------------------------
    float4_t o_acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o_acc[db] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = NEG_INF, l_run = 0.0f;

    const int64_t plane = ((int64_t)b * a.Hkv + g) * a.S;
    const uint8_t* kcodes = a.kc + plane * ROWB;
    const uint8_t* vcodes = a.vc + plane * ROWB;
    // this workgroup's share of the key tiles (all of them unless the key
    // range is split over gridDim.y workgroups), cut at loop_end; t below
    // counts tiles from t0.  Split boundaries follow kv_len, not loop_end, so
    // skipping the tiles past the causal bound changes no boundary and stays
    // bit-identical to scanning them (they are fully masked and add 0).
    const int per_split = ((kv_len + BN - 1) / BN + a.kv_splits - 1) / a.kv_splits;
    const int t0 = (int)blockIdx.y * per_split;
    const int n_tiles = max(min(per_split, (loop_end + BN - 1) / BN - t0), 0);
    const int diag_lo = qpos0 + r0;        // keys <= this are visible to every row of the tile
    const int lim = a.causal ? qpos0 + q_row : kv_len - 1;   // this column's last visible key

    // Asynchronous copy of tile tt's code rows: waves 0-3 fetch K, waves 4-7 V,
    // 256 x 16 bytes per step.  The K tile goes part-major when an eighth of a
    // row is at least 16 bytes (so the K stage reads conflict-free), else
    // row-major like V.
    constexpr int RSTEPS = (TILEB + 4095) / 4096;
    static_assert(TILEB % 4096 == 0 || TILEB < 4096, "raw tile steps");
    auto fetch_raw = [&](int tt, uint8_t* raw) {
        const int jt = (t0 + tt) * BN;
        const uint8_t* src = vhalf ? vcodes : kcodes;
        uint8_t* dst = raw + (vhalf ? TILEB : 0);
#pragma unroll
        for (int i = 0; i < RSTEPS; ++i) {
            const int off = i * 4096 + t256 * 16;
            if (TILEB < 4096 && off >= TILEB) continue;   // whole waves past a small tile
            int key, col;
            if (KPM && !vhalf) {
                const int u = off / RB;
                key = u % BN;
                col = (u / BN) * RB + off % RB;
            } else {
                key = off / ROWB;
                col = off % ROWB;
            }
            const int64_t j = min(jt + key, kv_len - 1);   // rows below kv_len only
            __attribute__((address_space(3))) void* l =
                (__attribute__((address_space(3))) void*)(dst + i * 4096 + (wave & 3) * 1024);
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + j * ROWB + col),
                                             l, 16, 0, 0);
        }
    };
    float mk_s = 0.0f, mv_s = 0.0f;
    int mk_z = 0, mv_z = 0;
    uint32_t bk_r = 0, bv_r = 0;                      // block scales as loaded (fp32 bits / E8M0)
    auto fetch_meta = [&](int tt) {
        if constexpr (BLK) {
            if (tid < NG * BN) {                      // thread -> (group tid / BN, key tid % BN)
                const int j = min((t0 + tt) * BN + tid % BN, kv_len - 1);
                const int64_t gi = (plane + j) * NG + tid / BN;
                if constexpr (SC8) {
                    bk_r = reinterpret_cast<const uint8_t*>(a.ks)[gi];
                    bv_r = reinterpret_cast<const uint8_t*>(a.vs)[gi];
                } else {
                    bk_r = reinterpret_cast<const uint32_t*>(a.ks)[gi];
                    bv_r = reinterpret_cast<const uint32_t*>(a.vs)[gi];
                }
            }
        } else if (tid < BN) {
            const int j = min((t0 + tt) * BN + tid, kv_len - 1);
            mk_s = a.ks[plane + j];
            mv_s = a.vs[plane + j];
            mk_z = a.kz[plane + j];
            mv_z = a.vz[plane + j];
        }
    };
    auto blk_scale = [](uint32_t raw) {              // E8M0 b = 2^(b - 127), b = 0 the subnormal 2^-127
        if constexpr (SC8) return __uint_as_float(raw ? raw << 23 : 0x00400000u);
        else return __uint_as_float(raw);
    };
    auto store_meta = [&](int buf) {
        if constexpr (BLK) {
            if (tid < NG * BN) {
                const int gk = (tid / BN) * BN + tid % BN;
                bks_lds[buf][gk] = blk_scale(bk_r);
                bvs_lds[buf][gk] = blk_scale(bv_r);
            }
        } else if (tid < BN) {
            mks_lds[buf][tid] = mk_s;
            mvs_lds[buf][tid] = mv_s;
            mkz_lds[buf][tid] = mk_z;
            mvz_lds[buf][tid] = mv_z;
        }
    };

    // Dequantize tile tt (raw codes in raw, metadata in mbuf) into the fp16
    // tiles kt / vt, its K scales (times the q rescale) into ct, and into sv
    // each key's V scale (block caches, masked calls only: the largest of its
    // row's block scales), 0 past kv_len.
    auto stage = [&](auto vh, int tt, const uint8_t* raw, int mbuf, _Float16* kt, _Float16* vt, float* ct, float* sv,
                     float* bkt, float* bvt) __attribute__((always_inline)) {
        constexpr bool VH = decltype(vh)::value;
        if constexpr (!VH) {
            // thread -> (key, eighth of the row: D/8 elements)
            constexpr int NPR = D / 16;                    // fp16 pairs of an eighth
            const int key = KPM ? (t256 & 31) : (t256 >> 3);
            const int part = KPM ? (t256 >> 5) : (t256 & 7);
            const uint8_t* rk = raw + (KPM ? (part * BN + key) * RB : key * ROWB + part * RB);
            const uint32_t off = BLK ? 0u : zp_pair(mkz_lds[mbuf][key], U4);
            uint32_t w[RB / 4];
#pragma unroll
            for (int i = 0; i < RB / 4; ++i) w[i] = reinterpret_cast<const uint32_t*>(rk)[i];
            uint32_t hv[NPR];
#pragma unroll
            for (int i = 0; i < RB / 4; ++i) {
                if constexpr (BLK) blk_dword<QM>(w[i], hv + (F4 ? 4 : 2) * i);
                else if constexpr (U4) dq_dword_u4p(w[i], off, hv + 4 * i);
                else dq_dword_i8(w[i], off, hv + 2 * i);
            }
            constexpr int CPP = D / 64;                    // 16-byte chunks of an eighth
#pragma unroll
            for (int c = 0; c < CPP; ++c) {
                const int ch = (part * CPP + c) ^ pf_ksw<D>(key);
                *reinterpret_cast<uint4*>(kt + key * D + ch * 8) =
                    make_uint4(hv[4 * c], hv[4 * c + 1], hv[4 * c + 2], hv[4 * c + 3]);
            }
            if constexpr (BLK) {
                // block scales of keys past kv_len become 0 (their P is 0 too)
                if (tid < NG * BN) {
                    const bool in = (t0 + tt) * BN + tid % BN < kv_len;
                    bkt[tid] = in ? bks_lds[mbuf][tid] : 0.0f;
                    bvt[tid] = in ? finite_or_0(bvs_lds[mbuf][tid]) : 0.0f;
                }
                if (tid < BN) {
                    const bool in = (t0 + tt) * BN + tid < kv_len;
                    ct[tid] = in ? rs : 0.0f;
                    if (has_mask) {                        // the masked path's V-scale bound
                        float mx = 0.0f;
#pragma unroll
                        for (int gg = 0; gg < NG; ++gg) mx = fmaxf(mx, bvs_lds[mbuf][gg * BN + tid]);
                        sv[tid] = in ? mx : 0.0f;
                    }
                }
            } else if (tid < BN) {
                const bool in = (t0 + tt) * BN + tid < kv_len;
                ct[tid] = in ? mks_lds[mbuf][tid] * rs : 0.0f;
                sv[tid] = in ? finite_or_0(mvs_lds[mbuf][tid]) : 0.0f;
            }
        } else {
            // thread -> (8 d, 4 keys); consecutive threads take consecutive d
            // groups, so the raw reads and the V^T row stores are contiguous
            const int dg = t256 % DG, kg = t256 / DG;
            if (kg < BN / 4) {
                const uint8_t* rv = raw + TILEB;
                uint32_t pr[4][4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int k = kg * 4 + e;
                    const uint32_t offv = BLK ? 0u : zp_pair(mvz_lds[mbuf][k], U4);
                    const uint8_t* vs = rv + k * ROWB + (U4 ? dg * 4 : dg * 8);
                    if constexpr (BLK) {
                        if constexpr (F4) {
                            blk_dword<QM>(*reinterpret_cast<const uint32_t*>(vs), pr[e]);
                        } else {
                            const uint2 w2 = *reinterpret_cast<const uint2*>(vs);
                            blk_dword<QM>(w2.x, pr[e]);
                            blk_dword<QM>(w2.y, pr[e] + 2);
                        }
                    } else if constexpr (U4) {
                        dq_dword_u4p(*reinterpret_cast<const uint32_t*>(vs), offv, pr[e]);
                    } else {
                        const uint2 w2 = *reinterpret_cast<const uint2*>(vs);
                        dq_dword_i8(w2.x, offv, pr[e]);
                        dq_dword_i8(w2.y, offv, pr[e] + 2);
                    }
                }
                const int col0 = pf_col(kg * 4);          // 4 consecutive columns
#pragma unroll
                for (int dd = 0; dd < 8; ++dd) {
                    const int pq = PERM ? ((dd & 1) * 2 + (dd >> 2)) : (dd >> 1);
                    const int ph = PERM ? ((dd >> 1) & 1) : (dd & 1);
                    const uint32_t sel = ph ? 0x07060302u : 0x05040100u;
                    const uint32_t w0 = __builtin_amdgcn_perm(pr[1][pq], pr[0][pq], sel);
                    const uint32_t w1 = __builtin_amdgcn_perm(pr[3][pq], pr[2][pq], sel);
                    const int row = BLK ? dg * 8 + dd : dd * DG + dg;   // R(d) for d = dg * 8 + dd
                    const int ch = (col0 >> 3) ^ (BLK ? pf_vswb(row) : pf_vsw(row));
                    *reinterpret_cast<uint2*>(vt + row * BN + ch * 8 + (col0 & 7)) = make_uint2(w0, w1);
                }
            }
        }
    };

    // ---- no mask: log2 of the largest V scale of this workgroup's keys -----
    // (block caches: of all their block scales); a per-wave maximum now, the
    // workgroup's after the prologue's barrier.  The range is the split's
    // share below kv_len, not cut at the causal bound, so skipping the tiles
    // past that bound still changes no bit.
    __shared__ float vb_lds[PF_WAVES];
    float lsv_wg = PF_LSV_MIN;
    if (!has_mask && n_tiles > 0) {
        const int k0 = t0 * BN, k1 = min(kv_len, (t0 + per_split) * BN);
        float x = 0.0f;
        if constexpr (BLK) {
            const int64_t g0 = (plane + k0) * NG;
            const int cnt = (k1 - k0) * NG;
            if constexpr (SC8) {
                // E8M0 bytes: 16 at a time where aligned (the order of the
                // codes is the order of the scales)
                const uint8_t* vb = reinterpret_cast<const uint8_t*>(a.vs) + g0;
                const int h = min((int)((16 - ((uintptr_t)vb & 15)) & 15), cnt);
                uint32_t mb = tid < h ? vb[tid] : 0u;
                const uint4* v16 = reinterpret_cast<const uint4*>(vb + h);
                const int n16 = (cnt - h) / 16;
#pragma unroll 16
                for (int i = tid; i < n16; i += 64 * PF_WAVES) {
                    const uint4 w4 = v16[i];
                    const uint32_t ws[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        mb = max(mb, max(max(ws[k] & 0xFFu, (ws[k] >> 8) & 0xFFu),
                                         max((ws[k] >> 16) & 0xFFu, ws[k] >> 24)));
                }
                const int tl = h + n16 * 16;
                if (tid < cnt - tl) mb = max(mb, (uint32_t)vb[tl + tid]);
                x = mb ? blk_scale(mb) : 0.0f;
            } else {
                x = range_max_f32(a.vs + g0, cnt, tid);
            }
        } else {
            x = range_max_f32(a.vs + plane + k0, k1 - k0, tid);
        }
        // wave maximum: within quads (xor 1, xor 2), half rows and rows
        // (mirrors), then across rows (lanes l^16, l^32)
        x = fmaxf(x, dpp_f32<0xB1>(x));
        x = fmaxf(x, dpp_f32<0x4E>(x));
        x = fmaxf(x, dpp_f32<0x141>(x));
        x = fmaxf(x, dpp_f32<0x140>(x));
        auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
        auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
        if (lane == 0) vb_lds[wave] = x;
    }

    // ---- prologue: tiles 0 and 1 in flight, tile 0 dequantized ---------------
    if (n_tiles > 0) {
        fetch_meta(0);
        fetch_raw(0, raw_a);
        store_meta(0);
        if (n_tiles > 1) {
            fetch_meta(1);
            fetch_raw(1, raw_b);
            store_meta(1);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (!has_mask) {
            float x = 0.0f;
#pragma unroll
            for (int w = 0; w < PF_WAVES; ++w) x = fmaxf(x, vb_lds[w]);
            lsv_wg = fmaxf(__builtin_amdgcn_logf(x), PF_LSV_MIN);
        }
        if (vhalf) stage(std::true_type{}, 0, raw_a, 0, k_a, v_a, c_a, s_a, bk_a, bv_a);
        else stage(std::false_type{}, 0, raw_a, 0, k_a, v_a, c_a, s_a, bk_a, bv_a);
        __syncthreads();
    }

    // Tile t: computes on (kc, vc, cc, sc); dequantizes tile t+1 from raw_n1
    // into (kn, vn, cn, sn); streams tile t+2 into raw_n2 (the buffer tile t
    // came through).
    auto tile = [&](auto vh, const int t, const _Float16* kc, const _Float16* vc, const float* cc, const float* sc,
                    const float* bkc, const float* bvc, _Float16* kn, _Float16* vn, float* cn, float* sn,
                    float* bkn, float* bvn, const uint8_t* raw_n1, uint8_t* raw_n2) __attribute__((always_inline)) {
        const int j0 = (t0 + t) * BN;
        if (t + 2 < n_tiles) {
            fetch_meta(t + 2);
            fetch_raw(t + 2, raw_n2);
        }
        // ---------------- S^T = K Q^T for the two 16-key blocks ----------------
        float4_t st[2] = {float4_t{0.0f, 0.0f, 0.0f, 0.0f}, float4_t{0.0f, 0.0f, 0.0f, 0.0f}};
        if constexpr (BLK) {
            // one k-step = one 32-element scale block: each block's partial
            // product is scaled per key (the lane's 4 keys) and summed in fp32;
            // block by block, so only two partials are live at a time
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) {
                float4_t part[2];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int key = kb * 16 + l16;
                    const int ch = (ds * 4 + lg) ^ pf_ksw<D>(key);
                    const half8_t av = *reinterpret_cast<const half8_t*>(kc + key * D + ch * 8);
                    part[kb] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int ql = 0; ql < QL; ++ql)
                        part[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qh[ds][ql], part[kb], 0, 0, 0);
                }
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const float4 k4 = *reinterpret_cast<const float4*>(bkc + ds * BN + kb * 16 + 4 * lg);
                    st[kb][0] = fmaf(part[kb][0], k4.x, st[kb][0]);
                    st[kb][1] = fmaf(part[kb][1], k4.y, st[kb][1]);
                    st[kb][2] = fmaf(part[kb][2], k4.z, st[kb][2]);
                    st[kb][3] = fmaf(part[kb][3], k4.w, st[kb][3]);
                }
                // keep the scaling here: sunk to the softmax it would hold
                // every block's partial across the stage of the next tile
                asm volatile("" : "+v"(st[0]), "+v"(st[1]));
            }
        } else {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int key = kb * 16 + l16;
#pragma unroll
                for (int ds = 0; ds < NDS; ++ds) {
                    const int ch = (ds * 4 + lg) ^ pf_ksw<D>(key);
                    const half8_t av = *reinterpret_cast<const half8_t*>(kc + key * D + ch * 8);
#pragma unroll
                    for (int ql = 0; ql < QL; ++ql)
                        st[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qh[ds][ql], st[kb], 0, 0, 0);
                }
            }
        }
        // ---------------- tile t+1 dequantized while those MFMAs run -----------
        // (unconditional, so it stays in the MFMAs' basic block: past the last
        // tile it converts whatever the raw buffer holds into a buffer nobody
        // reads)
        stage(vh, t + 1, raw_n1, (t + 1) & 1, kn, vn, cn, sn, bkn, bvn);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // four VALU
        }

        // ---------------- softmax over this lane's 8 keys -----------------------
        // lane holds keys j0 + kb*16 + 4*lg + i of query column qc
        const bool tile_mask = (a.causal && j0 + BN - 1 > diag_lo) || (j0 + BN > kv_len) || has_mask || !q_live;
        float sv8[8];
        float tmax = NEG_INF;
        uint32_t hid = 0;                                  // keys the mask hides from this column
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const float4 c4 = *reinterpret_cast<const float4*>(cc + kb * 16 + 4 * lg);
            const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = st[kb][i] * cv[i];
                if (tile_mask) {
                    const int key = j0 + kb * 16 + 4 * lg + i;
                    if (has_mask && key < kv_len && q_live) {
                        // a masked key is -inf whatever its (possibly unwritten) scale holds
                        const float mv = a.mask[(int64_t)q_row * a.S + key];
                        v = mv == NEG_INF ? NEG_INF : v + mv * 1.4426950408889634f;
                        if (mv == NEG_INF) hid |= 1u << (kb * 4 + i);
                    }
                    if (key > lim || key >= kv_len || !q_live) v = NEG_INF;
                }
                sv8[kb * 4 + i] = v;
                tmax = fmaxf(tmax, v);
            }
        }
        // max over the 4 lane groups of this column (lanes l, l^16, l^32, l^48)
        {
            auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
            tmax = fmax_q(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
            auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
            tmax = fmax_q(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
        }
        // log2 of the largest V scale the column may weight in this tile
        float lsv;
        if (has_mask) {
            float vmax = 0.0f;                             // staged 0 past kv_len
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const float4 v4 = *reinterpret_cast<const float4*>(sc + kb * 16 + 4 * lg);
                const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) vmax = fmaxf(vmax, (hid >> (kb * 4 + i)) & 1u ? 0.0f : vv[i]);
            }
            auto w32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(vmax), __float_as_uint(vmax), false, false);
            vmax = fmaxf(__uint_as_float(w32[0]), __uint_as_float(w32[1]));
            auto w16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(vmax), __float_as_uint(vmax), false, false);
            vmax = fmaxf(__uint_as_float(w16[0]), __uint_as_float(w16[1]));
            lsv = fmaxf(__builtin_amdgcn_logf(vmax), PF_LSV_MIN);
        } else {
            lsv = lsv_wg;
        }
        // bound on log2(p' * scale_v) over the tile, less m_run
        const float bnd = tmax + lsv;
        const bool upd = bnd > m_run + PF_PV_HI;
        if (__any(upd)) {
            const float mn = upd ? bnd - PF_PV_SET : m_run;
            const float al = m_run == NEG_INF ? 0.0f : __builtin_amdgcn_exp2f(m_run - mn);
            m_run = mn;
            l_run *= al;
#pragma unroll
            for (int db = 0; db < NDB; ++db) o_acc[db] *= al;
        }
        const float msafe = m_run == NEG_INF ? 0.0f : m_run;
        float p8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            p8[e] = __builtin_amdgcn_exp2f(sv8[e] - msafe);
            l_run += p8[e];
        }
        // P * scale_v for the lane's 8 keys (scales sv[4lg..+3], sv[16+4lg..+3])
        // as hi (+ lo) fp16 limbs: the B operand of the PV product
        auto pack_p = [&](const float* svp, half8_t* pb) {
            const float4 s0 = *reinterpret_cast<const float4*>(svp + 4 * lg);
            const float4 s1 = *reinterpret_cast<const float4*>(svp + 16 + 4 * lg);
            const float svv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                // a dropped key (p = 0) adds exactly 0: its staged scale is finite
                const float pv0 = p8[e] * svv[e];
                const float pv1 = p8[e + 1] * svv[e + 1];
                const half2_t h2 = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(pv0, pv1));
                pb[0][e] = h2[0];
                pb[0][e + 1] = h2[1];
                if constexpr (PL == 2) {
                    const half2_t l2 = __builtin_bit_cast(
                        half2_t, __builtin_amdgcn_cvt_pkrtz(pv0 - (float)h2[0], pv1 - (float)h2[1]));
                    pb[PL - 1][e] = l2[0];
                    pb[PL - 1][e + 1] = l2[1];
                }
            }
        };

        // ---------------- O^T += V^T P^T ------------------------------------------
        if constexpr (BLK) {
            // rows in d order; output blocks 2g and 2g + 1 lie in scale block g
#pragma unroll
            for (int gb = 0; gb < NG; ++gb) {
                half8_t pb[PL];
                pack_p(bvc + gb * BN, pb);
#pragma unroll
                for (int db = 2 * gb; db < 2 * gb + 2; ++db) {
                    const int row = db * 16 + l16;
                    const int ch = lg ^ pf_vswb(row);
                    const half8_t av = *reinterpret_cast<const half8_t*>(vc + row * BN + ch * 8);
#pragma unroll
                    for (int pl = 0; pl < PL; ++pl)
                        o_acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pb[pl], o_acc[db], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);    // one group's P limbs live at a time
            }
        } else {
            // rows in the R(d) order
            half8_t pb[PL];
            pack_p(sc, pb);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const int row = db * 16 + l16;
                const int ch = lg ^ pf_vsw(row);
                const half8_t av = *reinterpret_cast<const half8_t*>(vc + row * BN + ch * 8);
#pragma unroll
                for (int pl = 0; pl < PL; ++pl)
                    o_acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pb[pl], o_acc[db], 0, 0, 0);
            }
        }
        if (t + 2 < n_tiles) store_meta(t & 1);       // tile t+2's metadata replaces tile t's
        __builtin_amdgcn_s_waitcnt(0);                // tile t+2's code rows have landed
        __syncthreads();
    };
    auto run = [&](auto vh) __attribute__((always_inline)) {
        for (int t = 0; t < n_tiles; t += 2) {
            tile(vh, t, k_a, v_a, c_a, s_a, bk_a, bv_a, k_b, v_b, c_b, s_b, bk_b, bv_b, raw_b, raw_a);
            if (t + 1 < n_tiles) tile(vh, t + 1, k_b, v_b, c_b, s_b, bk_b, bv_b, k_a, v_a, c_a, s_a, bk_a, bv_a, raw_a, raw_b);
        }
    };
    if (vhalf) run(std::true_type{});
    else run(std::false_type{});

    // ---- epilogue: l over the 4 lane groups, normalize, store --------------------
    {
        auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
        l_run = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
        auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
        l_run = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    }
    if (!q_live) return;
    if (a.kv_splits > 1) {
        // partial (m, l, o) of this key range for the split combine (o and l
        // both in units of 2^m)
        const int64_t pr = (((int64_t)b * a.Hq + q_head) * a.Lq + q_row) * a.kv_splits + blockIdx.y;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int R = db * 16 + 4 * lg + i;
                const int d = BLK ? R : (R % DG) * 8 + R / DG;
                a.part_o[pr * D + d] = o_acc[db][i];
            }
        }
        if (lg == 0) {
            a.part_ml[pr * 2] = m_run;
            a.part_ml[pr * 2 + 1] = l_run;
        }
        return;
    }
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    const int64_t obase = (((int64_t)b * a.Hq + q_head) * a.Lq + q_row) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int R = db * 16 + 4 * lg + i;
            const int d = BLK ? R : (R % DG) * 8 + R / DG;   // row R holds d with R(d) = R
            const float v = o_acc[db][i] * inv;
            if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[obase + d] = f32_to_bf16_rne(v);
            else reinterpret_cast<float*>(a.out)[obase + d] = v;
        }
    }
}

template <int D, int QM, int QL, int PL>
static hipError_t launch_pf(const PrefillArgs& a, hipStream_t s) {
    const int G = a.Hq / a.Hkv;
    const int QT = 16 * PF_WAVES / G;
    PrefillArgs aa = a;
    aa.n_qtiles = (a.Lq + QT - 1) / QT;
    const unsigned blocks = (unsigned)(a.B * a.Hkv * aa.n_qtiles);
    hipLaunchKernelGGL((sdpa_prefill_mfma<D, QM, QL, PL>), dim3(blocks, (unsigned)a.kv_splits), dim3(64 * PF_WAVES), 0, s,
                       aa);
    return hipGetLastError();
}

template <int D, int QM>
static hipError_t dispatch_pf(const PrefillArgs& a, bool q_bf16, hipStream_t s) {
    // bf16 queries: one fp16 limb for Q (exact); fp32 queries: hi + lo limbs.
    // P * scale_v always goes in as hi + lo fp16 limbs (about 22 bits).
    if (q_bf16) return launch_pf<D, QM, 1, 2>(a, s);
    return launch_pf<D, QM, 2, 2>(a, s);
}

template <int D>
static hipError_t dispatch_pm(const PrefillArgs& a, int qmode, bool q_bf16, hipStream_t s) {
    switch (qmode) {
    case QM_INT8_TH: return dispatch_pf<D, QM_INT8_TH>(a, q_bf16, s);
    case QM_UINT4_TH: return dispatch_pf<D, QM_UINT4_TH>(a, q_bf16, s);
    case QM_FP8E4M3_B32: return dispatch_pf<D, QM_FP8E4M3_B32>(a, q_bf16, s);
    case QM_MXFP4_B32: return dispatch_pf<D, QM_MXFP4_B32>(a, q_bf16, s);
    case QM_MXFP8_B32: return dispatch_pf<D, QM_MXFP8_B32>(a, q_bf16, s);
    case QM_FP8E5M2_B32: return dispatch_pf<D, QM_FP8E5M2_B32>(a, q_bf16, s);
    case QM_INT8_B32: return dispatch_pf<D, QM_INT8_B32>(a, q_bf16, s);
    case QM_MXFP4E1M2_B32: return dispatch_pf<D, QM_MXFP4E1M2_B32>(a, q_bf16, s);
    default: return hipErrorNotSupported;
    }
}

hipError_t launch_sdpa_prefill(const PrefillLaunch& L, hipStream_t s) {
    const int ks = L.kv_splits > 1 ? L.kv_splits : 1;
    PrefillArgs a{L.q, L.B, L.Hq, L.Hkv, L.S, L.Lq, 0, L.kc, L.ks, L.kz, L.vc, L.vs, L.vz, L.kv_len, L.kv_len_sb,
                  L.mask, L.causal ? 1 : 0, L.no_skip ? 1 : 0, L.out_bf16 ? 1 : 0,
                  L.sm_scale * 1.4426950408889634f, L.out, L.err, ks, L.part_o, L.part_ml};
    const int G = L.Hq / L.Hkv;
    if (G < 1 || G > 8 || (G & (G - 1))) return hipErrorNotSupported;
    if (ks > 1 && (!L.part_o || !L.part_ml)) return hipErrorInvalidValue;
    hipError_t e;
    switch (L.D) {
    case 64: e = dispatch_pm<64>(a, L.qmode, L.q_bf16, s); break;
    case 128: e = dispatch_pm<128>(a, L.qmode, L.q_bf16, s); break;
    case 256: e = dispatch_pm<256>(a, L.qmode, L.q_bf16, s); break;
    default: return hipErrorNotSupported;
    }
    if (e != hipSuccess || ks == 1) return e;
    return launch_split_combine(L.D, L.part_o, L.part_ml, ks, (int64_t)L.B * L.Hq * L.Lq, L.out, L.out_bf16, s);
}

// Key-range splits of a prefill launch: enough workgroups for one per CU of
// the 256 -- one round, as the kernels keep one 8-wave workgroup per CU;
// measured faster than two or more rounds, whose extra splits add partials
// to write and merge -- for a chunk whose query tiles alone give fewer, each
// split covering at least 8 key tiles (256 keys) of the n_slots upper bound,
// at most 64.  1 when the query tiles already fill the part.  The same on
// every device, so the workspace size can be queried without one.
int prefill_kv_splits(int B, int Hq, int Hkv, int Lq, int S) {
    const int G = Hq / Hkv;
    if (G < 1) return 1;
    const int QT = 16 * PF_WAVES / G;
    const int64_t blocks = (int64_t)B * Hkv * ((Lq + QT - 1) / QT);
    if (blocks >= 256) return 1;
    int ks = (int)((256 + blocks - 1) / blocks);
    const int by_len = (S + 8 * PF_BN - 1) / (8 * PF_BN);
    if (ks > by_len) ks = by_len;
    if (ks > 64) ks = 64;
    return ks < 1 ? 1 : ks;
}

}  // namespace kvq
