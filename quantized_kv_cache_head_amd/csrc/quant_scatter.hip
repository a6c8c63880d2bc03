// quant_scatter.hip -- quantize new K/V vectors and scatter them to cache slots.
//
// Affine per token-head modes (int8 and 4-bit): pytorch/executorch PR 24473
// (Summary: int8 entries per token and head, affine asymmetric, float32 scale,
// int8 zero point, written through slot indices) and PR 20351 (4-bit codes
// packed two per byte along head_dim; static scatter along the position dim).
// Block modes (32 elements per block): IndexerQuantCache page, function
// description (scale = max|x_g| / Q_MAX, q = round(x / scale); the MX-FP8 and
// MX-FP4 modes with an E8M0 scale, the Normal mode with an fp32 scale),
// parameter table (FP8-E4M3FN, FP8-E5M2 and UINT8 caches; round_scale) and
// constraints (slot -1 skipped, valid slots in [0, num_slots)).
//
// Affine rule (the pages name the scheme without a formula; this is the
// reading the library implements): lo = min(0, min x), hi = max(0, max x),
// scale = max((hi - lo) / (qmax - qmin), 2^-23), zp = clamp(qmin -
// rne(lo / scale)), code = clamp(rne(x / scale) + zp).  Q_MAX: 448 (E4M3),
// 57344 (E5M2), 127 (int8, symmetric codes in [-127, 127]), 6 (E2M1).  MX
// scale: the smallest power of two >= amax / Q_MAX, or with the OCP option
// 2^(floor(log2 amax) - emax) and saturation past Q_MAX.
//
// Work mapping: a row (one token of one head) is split over L lanes of a
// wavefront, 8 elements per lane (one 16-byte bf16 load), so a wave covers
// 64/L rows and the min/max reduction stays inside the row's lanes.  Each lane
// writes its 8 codes (8 or 4 bytes) in one store; the L lanes of a row write
// the contiguous code row.  Block modes: 4 lanes per 32-element block.
// All arithmetic is single IEEE fp32 operations (file built with
// -ffp-contract=off; rintf is RNE), and every quotient is the correctly
// rounded one (a division, or a product shown to round to the same result),
// so codes, scales and zero points are bit-exact with the documented formulas.  FP8 and
// E2M1 codes come from the conversion instructions, which round the quotient
// to nearest even after a magnitude clamp (kvq_device.h).  An MX
// scale X = 2^k divides by multiplying with 2^-k, which is exactly
// representable (a subnormal for k = 127), so x * 2^-k rounds the same real
// number as x / X and gives the same bits.
//
// Latency: a lane issues its x load together with its slot load (a row whose
// slot turns out to be -1 has read 16 bytes for nothing), and thread indices
// become (b, h, t, lane) with 32-bit multiply-shift division by the host's
// precomputed constants (the launch holds fewer than 2^31 lanes).
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

// n / d for n < 2^31 as (umulhi(n, m) + n) >> s with s = ceil(log2 d) and
// m = floor(2^32 (2^s - d) / d) + 1 (Granlund and Montgomery, division by
// invariant integers using multiplication); the sum stays below 2^32.
struct FastDiv {
    uint32_t m, s;
};
static FastDiv make_fastdiv(uint32_t d) {
    uint32_t s = 0;
    while (s < 32 && (1ull << s) < d) ++s;
    return FastDiv{(uint32_t)((((1ull << s) - d) << 32) / d + 1), s};
}
__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) { return (__umulhi(n, f.m) + n) >> f.s; }

struct ScatterArgs {
    const void* x;
    int B, H, T, D;
    int64_t sb, sh, st;
    const int32_t* slots;
    int64_t ssb;
    int n_slots;
    uint8_t* codes;
    void* scales;
    int8_t* zps;
    int32_t* err;
    int flags;             // QF_MX_SCALE_OCP for the MX modes
    uint32_t rows;         // B * H * T
    FastDiv div_t, div_h, div_lpr;   // by T, by H, by the lanes of a row (block modes: D / 8)
    const int32_t* start_pos;        // non-null: slot = *start_pos + t (full-context layout), slots unused
    int off32;             // every element / byte offset of the launch fits in 31 bits (set by the host)
};

// The slot of token t: from the slot mapping, or (full-context layout) the
// position *start_pos + t itself, as kvq_positions_full gives it: a negative
// start writes nothing and sets the slot-range flag, a position past the
// cache writes nothing and sets the capacity flag.  report: the one lane of
// the row that may set flags.
__device__ __forceinline__ int token_slot(const ScatterArgs& a, int b, int t, bool report) {
    if (!a.start_pos) {
        if (a.off32) return a.slots[(uint32_t)b * (uint32_t)a.ssb + (uint32_t)t];
        return a.slots[(int64_t)b * a.ssb + t];
    }
    const int start = *a.start_pos;
    if (start < 0) {
        if (report && t == 0 && a.err) atomicOr(a.err, KVQ_DEV_FLAG_SLOT_RANGE);
        return -1;
    }
    const int64_t p = (int64_t)start + t;
    if (p >= a.n_slots) {
        if (report && a.err) atomicOr(a.err, KVQ_DEV_FLAG_POS_CAPACITY);
        return -1;
    }
    return (int)p;
}

// Row index -> (b, h, t).
__device__ __forceinline__ void row_coords(const ScatterArgs& a, uint32_t row, int& b, int& h, int& t) {
    const uint32_t bh = fdiv(row, a.div_t);
    t = (int)(row - bh * (uint32_t)a.T);
    b = (int)fdiv(bh, a.div_h);
    h = (int)(bh - (uint32_t)b * (uint32_t)a.H);
}

// Kernels take two argument sets and serve the one blockIdx.y picks (K and V
// of one update in a single launch; a single cache passes the same set twice
// and launches one grid row).
template <int L, int NP, bool BF16, bool U4>
__global__ __launch_bounds__(256) void quant_scatter_affine(ScatterArgs a0, ScatterArgs a1) {
    const ScatterArgs a = blockIdx.y ? a1 : a0;
    constexpr int QMIN = U4 ? 0 : -128;
    constexpr int QMAX = U4 ? 15 : 127;
    const int lane = threadIdx.x & 63;
    const int li = lane % L;
    const uint32_t row = (blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64) * (64 / L) + lane / L;

    // The slot and the row's x are loaded together (zeros past the last row
    // or past D; zeros never change the range, which always contains 0).
    int b = 0, h = 0, t = 0, slot = -1;
    float v[NP][8];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int i = 0; i < 8; ++i) v[p][i] = 0.0f;
    if (row < a.rows) {
        row_coords(a, row, b, h, t);
        slot = token_slot(a, b, t, h == 0 && li == 0);
        // 32-bit offsets where the host found that they fit: the wide
        // multiplies are a large part of a short-lived wave's instructions
        int64_t xoff;
        if (a.off32) xoff = (uint32_t)b * (uint32_t)a.sb + (uint32_t)h * (uint32_t)a.sh + (uint32_t)t * (uint32_t)a.st;
        else xoff = (int64_t)b * a.sb + (int64_t)h * a.sh + (int64_t)t * a.st;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int d0 = (p * L + li) * 8;
            if (d0 < a.D) load8<BF16>(a.x, xoff + d0, v[p]);
        }
        if (slot < -1 || slot >= a.n_slots) {
            if (h == 0 && li == 0 && a.err) atomicOr(a.err, KVQ_DEV_FLAG_SLOT_RANGE);
            slot = -1;
        }
    }
    const bool valid = slot >= 0;
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int i = 0; i < 8; ++i) { lo = fminf(lo, v[p][i]); hi = fmaxf(hi, v[p][i]); }
    lo = wave_min_sub<L>(lo);
    hi = wave_max_sub<L>(hi);
    if (!valid) return;

    // The row's chain (range, scale, 1 / scale, zero point) is the critical
    // path of a short-lived wave, so none of it is a division.
    // scale = RN(range / n), n = qmax - qmin (255 or 15), as s0 = range *
    // RN(1 / n) and one residual step: for these n the result equals the
    // correctly rounded quotient for every finite range >= 0 (an exhaustive
    // check over all of them is a CPU test); an infinite range keeps inf.
    constexpr float NQ = (float)(QMAX - QMIN);
    constexpr float RNQ = 1.0f / NQ;
    const float range = hi - lo;
    const float s0 = range * RNQ;
    float scale = fmaf(fmaf(-s0, NQ, range), RNQ, s0);
    if (!(range < __builtin_huge_valf())) scale = range;
    scale = fmaxf(scale, 0x1p-23f);

    // inv ~ 1 / scale: v_rcp (1 ulp) and one Newton step, within
    // 2^-24 (1 + 2^-20) of 1 / scale; 0 for an infinite scale.
    float inv = __builtin_amdgcn_rcpf(scale);
    inv = fmaf(fmaf(-scale, inv, 1.0f), inv, inv);
    if (!(scale < __builtin_huge_valf())) inv = 0.0f;

    // rne(x / scale) from x * inv: the product is within 3.01 * 2^-24 |q| of
    // RN(x / scale), where |q| = |x| / scale < 256 (x lies in [lo, hi] and
    // scale >= RN(range / n)), so below 2^-14.4.  Where it lies more than 2^-13
    // from every half-integer, both round to the same integer; a value closer
    // than that (or a non-finite one) takes the exact quotient instead.
    constexpr float TIE_MARGIN = 0x1p-13f;
    int zp;
    {
        const float t = lo * inv;
        float k = rintf(t);
        if (!(fabsf(t - k) < 0.5f - TIE_MARGIN)) k = rintf(lo / scale);
        zp = min(max(QMIN - (int)k, QMIN), QMAX);
    }
    // cache row and the byte offset of its codes
    constexpr int RB_DIV = U4 ? 2 : 1;
    int64_t crow, cbyte;
    if (a.off32) {
        const uint32_t r = ((uint32_t)b * (uint32_t)a.H + (uint32_t)h) * (uint32_t)a.n_slots + (uint32_t)slot;
        crow = r;
        cbyte = r * (uint32_t)(a.D / RB_DIV);
    } else {
        crow = ((int64_t)b * a.H + h) * a.n_slots + slot;
        cbyte = crow * (a.D / RB_DIV);
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int d0 = (p * L + li) * 8;
        if (d0 >= a.D) break;
        int c[8];
        // per element, with the exact product x * inv inside one fused
        // operation (it lies even closer to RN(x / scale) than the rounded
        // product): y = RN(x * inv + 1.5 * 2^23 + zp) holds n + zp, n the
        // integer nearest x * inv, in its low mantissa bits (|n + zp| < 2^22);
        // n = y - (1.5 * 2^23 + zp) exactly, and r = RN(x * inv - n) tells how
        // far x * inv is from n
        // far x * inv is from n.  The clamp to [qmin, qmax] is a float median
        // on y (the bounds 1.5 * 2^23 + qmin / qmax are exact), and the code
        // is the low byte (nibble) of y's bits: 1.5 * 2^23 has none set.
        const float mz = 0x1.8p23f + (float)zp;
        constexpr float YLO = 0x1.8p23f + (float)QMIN, YHI = 0x1.8p23f + (float)QMAX;
        bool near_tie = false;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float y = fmaf(v[p][i], inv, mz);
            const float r = fmaf(v[p][i], inv, -(y - mz));
            near_tie |= !(fabsf(r) < 0.5f - TIE_MARGIN);
            c[i] = (int)(__float_as_uint(__builtin_amdgcn_fmed3f(y, YLO, YHI)) & (U4 ? 0xFu : 0xFFu));
        }
        if (near_tie) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                int q = (int)rintf(v[p][i] / scale) + zp;
                c[i] = min(max(q, QMIN), QMAX);
            }
        }
        if constexpr (U4) {
            uint32_t w = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) w |= (uint32_t)c[i] << (4 * i);
            *reinterpret_cast<uint32_t*>(a.codes + cbyte + d0 / 2) = w;
        } else {
            uint32_t w0 = 0, w1 = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                w0 |= ((uint32_t)c[i] & 0xFFu) << (8 * i);
                w1 |= ((uint32_t)c[4 + i] & 0xFFu) << (8 * i);
            }
            *reinterpret_cast<uint2*>(a.codes + cbyte + d0) = make_uint2(w0, w1);
        }
    }
    if (li == 0) {
        reinterpret_cast<float*>(a.scales)[crow] = scale;
        a.zps[crow] = (int8_t)zp;
    }
}

template <bool BF16, int QM>
__global__ __launch_bounds__(256) void quant_scatter_block(ScatterArgs a0, ScatterArgs a1) {
    const ScatterArgs a = blockIdx.y ? a1 : a0;
    const uint32_t gl = blockIdx.x * blockDim.x + threadIdx.x;
    const int gpr = a.D / 32;                      // blocks per row
    const uint32_t row = fdiv(gl, a.div_lpr);
    const int lr = (int)(gl - row * (uint32_t)(a.D / 8));   // lane within the row
    const int qi = lr & 3;                         // lane within the 32-block
    const int g = lr >> 2;
    const int d0 = g * 32 + qi * 8;

    // the slot and the row's x are loaded together
    int b = 0, h = 0, t = 0, slot = -1;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    if (row < a.rows) {
        row_coords(a, row, b, h, t);
        slot = token_slot(a, b, t, h == 0 && g == 0 && qi == 0);
        int64_t xoff;
        if (a.off32) xoff = (uint32_t)b * (uint32_t)a.sb + (uint32_t)h * (uint32_t)a.sh + (uint32_t)t * (uint32_t)a.st;
        else xoff = (int64_t)b * a.sb + (int64_t)h * a.sh + (int64_t)t * a.st;
        load8<BF16>(a.x, xoff + d0, v);
        if (slot < -1 || slot >= a.n_slots) {
            if (h == 0 && g == 0 && qi == 0 && a.err) atomicOr(a.err, KVQ_DEV_FLAG_SLOT_RANGE);
            slot = -1;
        }
    }
    const bool valid = slot >= 0;
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = wave_max_sub<4>(amax);
    if (!valid) return;

    int64_t crow;
    if (a.off32) crow = ((uint32_t)b * (uint32_t)a.H + (uint32_t)h) * (uint32_t)a.n_slots + (uint32_t)slot;
    else crow = ((int64_t)b * a.H + h) * a.n_slots + slot;
    // byte offset of the row's codes (32-bit where the launch's offsets fit)
    constexpr int RB_DIV = (QM == QM_MXFP4_B32 || QM == QM_MXFP4E1M2_B32) ? 2 : 1;
    const int64_t cbyte = a.off32 ? (int64_t)((uint32_t)crow * (uint32_t)(a.D / RB_DIV)) : crow * (a.D / RB_DIV);
    if constexpr (QM == QM_FP8E4M3_B32 || QM == QM_FP8E5M2_B32 || QM == QM_INT8_B32) {
        // fp32 scale amax / Q_MAX; an all-zero block stores scale 0, codes 0
        constexpr float QMAX = QM == QM_FP8E4M3_B32 ? 448.0f : QM == QM_FP8E5M2_B32 ? 57344.0f : 127.0f;
        const float scale = amax / QMAX;
        uint32_t w0 = 0, w1 = 0;
        if (scale != 0.0f) {
            float y[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = v[i] / scale;
            if constexpr (QM == QM_FP8E4M3_B32) {
                w0 = cvt4_e4m3fn(y);
                w1 = cvt4_e4m3fn(y + 4);
            } else if constexpr (QM == QM_FP8E5M2_B32) {
                w0 = cvt4_e5m2(y);
                w1 = cvt4_e5m2(y + 4);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t c = (uint32_t)(int)fminf(fmaxf(rintf(y[i]), -127.0f), 127.0f) & 0xFFu;
                    if (i < 4) w0 |= c << (8 * i);
                    else w1 |= c << (8 * (i - 4));
                }
            }
        }
        *reinterpret_cast<uint2*>(a.codes + cbyte + d0) = make_uint2(w0, w1);
        if (qi == 0) reinterpret_cast<float*>(a.scales)[crow * gpr + g] = scale;
    } else {
        // MX: E8M0 power-of-two scale X; x / X is exact
        constexpr bool E1M2 = QM == QM_MXFP4E1M2_B32;
        constexpr bool F4 = QM == QM_MXFP4_B32 || E1M2;
        constexpr int EMAX = E1M2 ? 1 : F4 ? 2 : 8;
        constexpr float QMAX = E1M2 ? 3.5f : F4 ? 6.0f : 448.0f;
        const uint32_t e8 = (a.flags & QF_MX_SCALE_OCP) ? e8m0_floor(amax, EMAX) : e8m0_ceil(amax / QMAX);
        const float inv = __uint_as_float(e8 == 254u ? 0x00400000u : (254u - e8) << 23);   // 1 / X, exact
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = v[i] * inv;
        if constexpr (F4) {
            *reinterpret_cast<uint32_t*>(a.codes + cbyte + d0 / 2) = E1M2 ? cvt8_e1m2(y) : cvt8_e2m1(y);
        } else {
            *reinterpret_cast<uint2*>(a.codes + cbyte + d0) = make_uint2(cvt4_e4m3fn(y), cvt4_e4m3fn(y + 4));
        }
        if (qi == 0) reinterpret_cast<uint8_t*>(a.scales)[crow * gpr + g] = (uint8_t)e8;
    }
}

template <int L, int NP, bool BF16, bool U4>
static hipError_t launch_affine(const ScatterArgs& a, const ScatterArgs& a1, int n, hipStream_t s) {
    const int64_t rows = (int64_t)a.B * a.H * a.T;
    const int64_t rows_per_block = 4 * (64 / L);
    const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL((quant_scatter_affine<L, NP, BF16, U4>), dim3((unsigned)blocks, (unsigned)n), dim3(256), 0, s,
                       a, a1);
    return hipGetLastError();
}

template <bool BF16, bool U4>
static hipError_t dispatch_affine(const ScatterArgs& a, const ScatterArgs& a1, int n, hipStream_t s) {
    switch (a.D) {
    case 64: return launch_affine<8, 1, BF16, U4>(a, a1, n, s);
    case 128: return launch_affine<16, 1, BF16, U4>(a, a1, n, s);
    case 256: return launch_affine<32, 1, BF16, U4>(a, a1, n, s);
    case 512: return launch_affine<64, 1, BF16, U4>(a, a1, n, s);
    default:
        if (a.D <= 1024) return launch_affine<64, 2, BF16, U4>(a, a1, n, s);
        if (a.D <= 2048) return launch_affine<64, 4, BF16, U4>(a, a1, n, s);
        return launch_affine<64, 16, BF16, U4>(a, a1, n, s);
    }
}

// The launch's 32-bit index arithmetic needs fewer than 2^31 lanes (D / 8 per
// row; the affine kernels use at most that many).
static bool fill_index(ScatterArgs& a) {
    const int64_t rows = (int64_t)a.B * a.H * a.T;
    if (rows * ((a.D + 7) / 8) >= (int64_t(1) << 31)) return false;
    a.rows = (uint32_t)rows;
    a.div_t = make_fastdiv((uint32_t)a.T);
    a.div_h = make_fastdiv((uint32_t)a.H);
    a.div_lpr = make_fastdiv((uint32_t)(a.D / 8));
    // 32-bit offsets: x elements, slot entries and cache bytes (D per row
    // bounds the code bytes and the scale / zero-point entries) below 2^31
    const int64_t lim = int64_t(1) << 31;
    const int64_t xmax = (int64_t)(a.B - 1) * a.sb + (int64_t)(a.H - 1) * a.sh + (int64_t)(a.T - 1) * a.st + a.D;
    const int64_t smax = a.start_pos ? 0 : (int64_t)(a.B - 1) * a.ssb + a.T;
    const int64_t cmax = (int64_t)a.B * a.H * a.n_slots * a.D;
    a.off32 = a.sb >= 0 && a.sh >= 0 && a.st >= 0 && (a.start_pos || a.ssb >= 0) && xmax < lim && smax < lim &&
              cmax < lim;
    return true;
}

// One or two caches (n = 1 or 2) of the same mode and sizes in one launch.
static hipError_t launch_scatter_n(int qmode, bool bf16, ScatterArgs a, ScatterArgs a1, int n, hipStream_t s) {
    if (!fill_index(a) || !fill_index(a1)) return hipErrorInvalidValue;
    if (qmode == QM_INT8_TH) return bf16 ? dispatch_affine<true, false>(a, a1, n, s) : dispatch_affine<false, false>(a, a1, n, s);
    if (qmode == QM_UINT4_TH) return bf16 ? dispatch_affine<true, true>(a, a1, n, s) : dispatch_affine<false, true>(a, a1, n, s);
    const int64_t lanes = (int64_t)a.B * a.H * a.T * (a.D / 8);
    const dim3 grid((unsigned)((lanes + 255) / 256), (unsigned)n);
#define KVQ_BLK(QQ)                                                                                     \
    if (bf16) hipLaunchKernelGGL((quant_scatter_block<true, QQ>), grid, dim3(256), 0, s, a, a1);         \
    else hipLaunchKernelGGL((quant_scatter_block<false, QQ>), grid, dim3(256), 0, s, a, a1);
    switch (qmode) {
    case QM_FP8E4M3_B32: KVQ_BLK(QM_FP8E4M3_B32) break;
    case QM_MXFP4_B32: KVQ_BLK(QM_MXFP4_B32) break;
    case QM_MXFP4E1M2_B32: KVQ_BLK(QM_MXFP4E1M2_B32) break;
    case QM_MXFP8_B32: KVQ_BLK(QM_MXFP8_B32) break;
    case QM_FP8E5M2_B32: KVQ_BLK(QM_FP8E5M2_B32) break;
    case QM_INT8_B32: KVQ_BLK(QM_INT8_B32) break;
    default: return hipErrorInvalidValue;
    }
#undef KVQ_BLK
    return hipGetLastError();
}

hipError_t launch_quant_scatter(int qmode, bool bf16, const void* x, int B, int H, int T, int D,
                                int64_t sb, int64_t sh, int64_t st, const int32_t* slots,
                                int64_t ssb, int n_slots, uint8_t* codes, void* scales,
                                int8_t* zps, int flags, int32_t* err, hipStream_t s) {
    const ScatterArgs a{x, B, H, T, D, sb, sh, st, slots, ssb, n_slots, codes, scales, zps, err, flags, 0, {}, {}, {},
                        nullptr};
    return launch_scatter_n(qmode, bf16, a, a, 1, s);
}

hipError_t launch_quant_scatter_kv(int qmode, bool bf16, const void* xk, const void* xv, int B, int H, int T, int D,
                                   int64_t sb, int64_t sh, int64_t st, const int32_t* slots, int64_t ssb,
                                   int n_slots, uint8_t* kcodes, void* kscales, int8_t* kzps, uint8_t* vcodes,
                                   void* vscales, int8_t* vzps, const int32_t* start_pos, int32_t* err,
                                   hipStream_t s) {
    const ScatterArgs ak{xk, B, H, T, D, sb, sh, st, slots, ssb, n_slots, kcodes, kscales, kzps, err, 0, 0, {}, {}, {},
                         start_pos};
    const ScatterArgs av{xv, B, H, T, D, sb, sh, st, slots, ssb, n_slots, vcodes, vscales, vzps, err, 0, 0, {}, {}, {},
                         start_pos};
    return launch_scatter_n(qmode, bf16, ak, av, 2, s);
}

}  // namespace kvq
