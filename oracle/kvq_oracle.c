/*
 * kvq_oracle.c -- plain, slow CPU oracle for the quantized KV-cache hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline load it.  It shares no code, header, table or constant with the
 * HIP path.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC
 *   -ffp-contract=off : every fp32 step is one IEEE operation, no fused FMA.
 *   Default rounding mode (round to nearest even) is assumed throughout, so
 *   rintf() is round-half-to-even.
 *
 * Sources (the pages this oracle follows):
 *   [PR24473]   pytorch/executorch pull request 24473, "Summary": int8 entries
 *               quantized per token and head, affine asymmetric, float32 scales
 *               and int8 zero points; sink/ring slot layouts; additive float
 *               mask for ring/sink caches; plain causal attention otherwise.
 *   [PR20351]   pytorch/executorch pull request 20351 (gemma4_31b, CUDA
 *               backend), commit notes: 4-bit codes nibble-packed along the
 *               last dim, static scatter along the position dim, the kv_len
 *               bound on the KV loop, the per-tile causal upper bound.
 *   [IQC]       IndexerQuantCache operator page (ops-transformer): the
 *               per-block formula scale_g = max|x_g| / Q_MAX, q_i = round(x_i /
 *               scale_g) ("function description"), the parameter table, the
 *               constraints (slot -1 skipped, slots in [0, num_slots-1]).
 *   [ABADDON]   abaddon 0.2.0-rc.1, src/attention_cache/mod.rs: KvCache trait,
 *               K/V shape [batch, kv_heads, seq, head_dim], q/out shape
 *               [batch, heads, q_len, head_dim], forward_attention with GQA
 *               expansion (repeat_kv) and a softmax scale.
 *   [KVQC]      coreai_opt KVCacheQuantConfig: the cache op must commute with
 *               quantize/dequantize (pure data movement).
 *
 * Readings taken where the pages are silent:
 *   R1  int8/uint4 affine: range extended to include 0; zero point from the
 *       min side, zp = qmin - rne(lo/scale); codes clamp(rne(x/scale)+zp).
 *   R2  4-bit: unsigned codes 0..15, zero point 0..15 stored as int8, element
 *       2i in the low nibble of byte i.
 *   R3  scale floor 2^-23 so the scale is never 0 or subnormal.
 *   R4/R5 round half to even; IEEE correctly rounded fp32 division.
 *   R6  Q_MAX = 448 (E4M3FN), 6 (E2M1).
 *   R7  all-zero FP8 block: scale 0, codes 0x00.
 *   R8  saturate to +-Q_MAX; inputs are finite by contract.
 *   R9  MX-FP4 scale = smallest power of two >= amax/6 (E8M0, clamp [0,254]).
 *   R10 negative values that round to zero keep their sign bit.
 *   R11 mask: slot visible iff cp>=0, cp<=qp and (cp<sink or qp-cp<window).
 *   R13 a query row with no visible key outputs 0.
 *   R14 GQA: query head h reads KV head h / (Hq/Hkv).
 *   R22 Q_MAX = 57344 (E5M2, largest finite), 127 (INT8: symmetric codes in
 *       [-127, 127], two's complement in the uint8 cache).
 *   R23 MX-FP8 (quant_mode 0) with round_scale = true: the E8M0 scale is the
 *       smallest power of two >= amax / 448 (the same rounding as R9).
 *   R25 A call with more tokens than the ring holds writes them one after
 *       another: a token whose slot a later token of the call takes again is
 *       not written (slot -1); cache_positions keeps the last position.
 *   R24 round_scale = false, and the OCP variant of MX-FP4: the scale is
 *       2^(floor(log2 amax) - emax), emax = 8 (E4M3) or 2 (E2M1), clamped to
 *       the E8M0 range; elements beyond Q_MAX then saturate (R8).
 *   R27 FLOAT4_E1M2 (a cache dtype of the MX-FP4 mode on the IndexerQuantCache
 *       page, parameter table): sign, one exponent bit, two mantissa bits,
 *       exponent bias 0 (the IEEE rule 2^(k-1) - 1 for k = 1 exponent bit):
 *       exponent 0 is subnormal 0.mm x 2^1, exponent 1 is 1.mm x 2^1, so
 *       magnitude code c (0..7) is worth c / 2, Q_MAX = 3.5, emax = 1.  Under
 *       a power-of-two block scale any other bias only moves the stored E8M0
 *       exponent: the dequantized values stay the same.
 *
 * Parity pins: every function here is checked by the CPU tests against
 * closed forms, exhaustive grid search, library routines and hand-derived
 * worked examples.  The int8/uint4 affine formula family itself is fixed only
 * by reading R1 (the pages name the scheme but print no formula): that
 * choice of formula is "parity unpinned"; its properties are pinned.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

#define ORC_INT8_TH 0
#define ORC_UINT4_TH 1
#define ORC_FP8E4M3_B32 2
#define ORC_MXFP4_B32 3
#define ORC_MXFP8_B32 4     /* E4M3FN codes, E8M0 scale per 32 ([IQC] quant_mode 0) */
#define ORC_FP8E5M2_B32 5   /* E5M2 codes, fp32 scale per 32 ([IQC] Normal mode, E5M2 cache) */
#define ORC_INT8_B32 6      /* int8 codes in a uint8 cache, fp32 scale per 32 ([IQC] Normal, INT8) */
#define ORC_MXFP4E1M2_B32 7 /* FP4-E1M2 codes, E8M0 scale per 32 ([IQC] MX-FP4 mode, FLOAT4_E1M2 cache) */

/* Quantize option: the MX scale by the OCP floor rule (R24) instead of the
 * smallest power of two >= amax / Q_MAX (R9). */
#define ORC_MX_SCALE_OCP 1

#define ORC_FLAG_SLOT_RANGE 1   /* slot outside [-1, n_slots) */
#define ORC_FLAG_KVLEN 2        /* kv_len outside [Lq, n_slots] */
#define ORC_FLAG_POS_CAPACITY 4 /* full-context position >= n_slots */

/* ------------------------------------------------------------------------ */
/* Element encoders                                                          */
/* ------------------------------------------------------------------------ */

/* Largest finite magnitudes (reading R6). */
static const float E4M3_MAX = 448.0f;
static const float E2M1_MAX = 6.0f;
static const float E1M2_MAX = 3.5f;     /* R27 */

/* Unbiased exponent floor(log2 a) of a positive normal fp32 value. */
static int fp32_floor_log2(float a) {
    int e;
    frexpf(a, &e);          /* a = f * 2^e, f in [0.5, 1) */
    return e - 1;
}

/* FP8 E4M3FN: bias 7, 3 mantissa bits, subnormal step 2^-9, max 448, no inf.
 * Round to nearest with ties to the even mantissa; |y| >= 448 saturates to
 * 448 (R8); a negative value keeps its sign bit even when it rounds to 0
 * (R10).  [IQC] function description (FP8 target of the per-block formula). */
uint8_t orc_e4m3fn_encode(float y) {
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    float a = fabsf(y);
    uint8_t mag;
    if (!(a < E4M3_MAX)) {                 /* >= 448 (or inf): saturate */
        mag = 0x7E;
    } else if (a < 0x1p-6f) {              /* below the smallest normal */
        float m = rintf(a * 512.0f);       /* multiples of 2^-9, exact scale */
        mag = (uint8_t)m;                  /* m == 8 is the smallest normal */
    } else {
        int e = fp32_floor_log2(a);        /* -6 .. 8 */
        float frac = ldexpf(a, -e);        /* [1, 2), exact */
        float m = rintf((frac - 1.0f) * 8.0f);
        if (m == 8.0f) { m = 0.0f; e += 1; }
        mag = (uint8_t)(((e + 7) << 3) | (int)m);
        if (mag > 0x7E) mag = 0x7E;
    }
    return sign | mag;
}

float orc_e4m3fn_decode(uint8_t code) {
    int s = code >> 7, e = (code >> 3) & 0xF, m = code & 7;
    float v;
    if (e == 0xF && m == 7) return NAN;
    if (e == 0) v = ldexpf((float)m, -9);
    else v = ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return s ? -v : v;
}

/* FP4 E2M1: magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6} = codes 0..7, sign in bit
 * 3.  Nearest value, ties to the even code, |y| >= 6 saturates.  [IQC]
 * function description, MX-FP4 mode. */
uint8_t orc_e2m1_encode(float y) {
    uint8_t sign = signbit(y) ? 0x8 : 0x0;
    float a = fabsf(y);
    uint8_t mag;
    if (!(a < E2M1_MAX)) {
        mag = 7;
    } else if (a < 1.0f) {                 /* subnormal range, step 0.5 */
        mag = (uint8_t)rintf(a * 2.0f);    /* 2 is the smallest normal */
    } else {
        int e = fp32_floor_log2(a);        /* 0 .. 2 */
        float frac = ldexpf(a, -e);
        float m = rintf((frac - 1.0f) * 2.0f);
        if (m == 2.0f) { m = 0.0f; e += 1; }
        mag = (uint8_t)(((e + 1) << 1) | (int)m);
        if (mag > 7) mag = 7;
    }
    return sign | mag;
}

float orc_e2m1_decode(uint8_t code) {
    static const float mags[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    float v = mags[code & 7];
    return (code & 8) ? -v : v;
}

/* FP4 E1M2 (reading R27): bit 3 sign, bit 2 exponent, bits 1..0 mantissa.
 * Exponent 0: 0.mm x 2^1 (subnormal); exponent 1: 1.mm x 2^1. */
float orc_e1m2_decode(uint8_t code) {
    int e = (code >> 2) & 1, m = code & 3;
    float v = e ? ldexpf(1.0f + (float)m / 4.0f, 1) : ldexpf((float)m / 4.0f, 1);
    return (code & 8) ? -v : v;
}

/* Nearest E1M2 value, ties to the even code, |y| >= 3.5 saturates.  The
 * values 0, .5, ..., 3.5 are evenly spaced (the subnormal step 2^-1 equals
 * the normal one), so the nearest one to |y| is rne(2 |y|) / 2, and an even
 * code is an even mantissa. */
uint8_t orc_e1m2_encode(float y) {
    uint8_t sign = signbit(y) ? 0x8 : 0x0;
    float a = fabsf(y);
    uint8_t mag;
    if (!(a < E1M2_MAX)) mag = 7;
    else mag = (uint8_t)rintf(a * 2.0f);
    return sign | mag;
}

/* E8M0 scale for an MX block (reading R9): the smallest power of two that is
 * >= s, as a biased exponent clamped to [0, 254] (0xFF is NaN and never
 * produced).  ceil(log2 s) is read exactly from the fp32 bits of s. */
uint8_t orc_e8m0_ceil(float s) {
    if (!(s > 0.0f)) return 0;             /* s == 0: exponent -inf -> 0 */
    uint32_t bits;
    memcpy(&bits, &s, 4);
    int ef = (int)((bits >> 23) & 0xFF);
    uint32_t mant = bits & 0x7FFFFF;
    int E;
    if (ef == 0) {                         /* subnormal: s = mant * 2^-149 */
        int fl = 31 - __builtin_clz(mant); /* floor(log2 mant) */
        int pow2 = (mant & (mant - 1)) == 0;
        E = fl + (pow2 ? 0 : 1) - 149;
    } else {
        E = ef - 127 + (mant != 0 ? 1 : 0);
    }
    int b = E + 127;
    if (b < 0) b = 0;
    if (b > 254) b = 254;
    return (uint8_t)b;
}

float orc_e8m0_value(uint8_t b) { return ldexpf(1.0f, (int)b - 127); }

/* E8M0 by the OCP floor rule (R24): biased exponent floor(log2 amax) - emax
 * + 127, clamped to [0, 254]; amax == 0 gives 0.  floor(log2 amax) is read
 * exactly from the fp32 bits (normal or subnormal). */
uint8_t orc_e8m0_floor(float amax, int emax) {
    if (!(amax > 0.0f)) return 0;
    uint32_t bits;
    memcpy(&bits, &amax, 4);
    int ef = (int)((bits >> 23) & 0xFF);
    int fl = ef == 0 ? (31 - __builtin_clz(bits & 0x7FFFFF)) - 149 : ef - 127;
    int b = fl - emax + 127;
    if (b < 0) b = 0;
    if (b > 254) b = 254;
    return (uint8_t)b;
}

/* FP8 E5M2: bias 15, 2 mantissa bits, subnormal step 2^-16, largest finite
 * 57344; exponent 31 holds inf / NaN, which the encoder never produces
 * (|y| >= 57344 saturates to 0x7B, R8).  Ties to the even mantissa, sign
 * kept (R10).  [IQC] parameter table (FLOAT8_E5M2 cache). */
static const float E5M2_MAX = 57344.0f;
uint8_t orc_e5m2_encode(float y) {
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    float a = fabsf(y);
    uint8_t mag;
    if (!(a < E5M2_MAX)) {
        mag = 0x7B;
    } else if (a < 0x1p-14f) {             /* multiples of 2^-16 */
        mag = (uint8_t)rintf(a * 65536.0f);  /* 4 is the smallest normal */
    } else {
        int e = fp32_floor_log2(a);        /* -14 .. 15 */
        float frac = ldexpf(a, -e);
        float m = rintf((frac - 1.0f) * 4.0f);
        if (m == 4.0f) { m = 0.0f; e += 1; }
        mag = (uint8_t)(((e + 15) << 2) | (int)m);
        if (mag > 0x7B) mag = 0x7B;
    }
    return sign | mag;
}

float orc_e5m2_decode(uint8_t code) {
    int s = code >> 7, e = (code >> 2) & 0x1F, m = code & 3;
    float v;
    if (e == 31) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexpf((float)m, -16);
    else v = ldexpf(1.0f + (float)m / 4.0f, e - 15);
    return s ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* Affine per token-head quantization (O2; [PR24473] Summary; [PR20351]      */
/* nibble packing)                                                           */
/* ------------------------------------------------------------------------ */

static float affine_scale_floor(void) { return 0x1p-23f; }

/* Scale and zero point of one vector x[D] on the integer grid [qmin, qmax]. */
void orc_affine_params(const float* x, int D, int qmin, int qmax,
                       float* scale_out, int* zp_out) {
    float lo = 0.0f, hi = 0.0f;            /* range always contains 0 (R1) */
    for (int d = 0; d < D; ++d) {
        if (x[d] < lo) lo = x[d];
        if (x[d] > hi) hi = x[d];
    }
    float range = hi - lo;
    float scale = range / (float)(qmax - qmin);
    if (scale < affine_scale_floor()) scale = affine_scale_floor();   /* R3 */
    int zp = qmin - (int)rintf(lo / scale);
    if (zp < qmin) zp = qmin;
    if (zp > qmax) zp = qmax;
    *scale_out = scale;
    *zp_out = zp;
}

int orc_affine_code(float x, float scale, int zp, int qmin, int qmax) {
    int c = (int)rintf(x / scale) + zp;
    if (c < qmin) c = qmin;
    if (c > qmax) c = qmax;
    return c;
}

/* ------------------------------------------------------------------------ */
/* Cache row geometry                                                        */
/* ------------------------------------------------------------------------ */

static int row_bytes(int qmode, int D) {
    return (qmode == ORC_UINT4_TH || qmode == ORC_MXFP4_B32 || qmode == ORC_MXFP4E1M2_B32) ? D / 2 : D;
}
static int is_block(int qmode) { return qmode >= ORC_FP8E4M3_B32; }
static int e8m0_scales(int qmode) {
    return qmode == ORC_MXFP4_B32 || qmode == ORC_MXFP8_B32 || qmode == ORC_MXFP4E1M2_B32;
}
static int scales_per_row(int qmode, int D) {
    return is_block(qmode) ? D / 32 : 1;
}

int orc_row_bytes(int qmode, int D) { return row_bytes(qmode, D); }
int orc_scales_per_row(int qmode, int D) { return scales_per_row(qmode, D); }

/* Quantize one vector x[D] into one cache row: codes (row_bytes bytes),
 * scales (float[] for INT8/UINT4/FP8, uint8 E8M0[] for MX-FP4), zp. */
static void quantize_row(int qmode, int flags, const float* x, int D,
                         uint8_t* codes, void* scales, int8_t* zp_out) {
    if (qmode == ORC_INT8_TH || qmode == ORC_UINT4_TH) {
        int qmin = qmode == ORC_INT8_TH ? -128 : 0;
        int qmax = qmode == ORC_INT8_TH ? 127 : 15;
        float scale; int zp;
        orc_affine_params(x, D, qmin, qmax, &scale, &zp);
        ((float*)scales)[0] = scale;
        *zp_out = (int8_t)zp;
        if (qmode == ORC_INT8_TH) {
            for (int d = 0; d < D; ++d)
                codes[d] = (uint8_t)(int8_t)orc_affine_code(x[d], scale, zp, qmin, qmax);
        } else {
            for (int i = 0; i < D / 2; ++i) {
                int c0 = orc_affine_code(x[2 * i], scale, zp, qmin, qmax);
                int c1 = orc_affine_code(x[2 * i + 1], scale, zp, qmin, qmax);
                codes[i] = (uint8_t)(c0 | (c1 << 4));           /* R2 */
            }
        }
        return;
    }
    /* Per-32-element block modes ([IQC] function description). */
    for (int g = 0; g < D / 32; ++g) {
        const float* xg = x + 32 * g;
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i) {
            float a = fabsf(xg[i]);
            if (a > amax) amax = a;
        }
        if (qmode == ORC_FP8E4M3_B32 || qmode == ORC_FP8E5M2_B32 || qmode == ORC_INT8_B32) {
            /* fp32 scale = amax / Q_MAX; an all-zero block stores scale 0 and
             * codes 0 (R7) */
            float qmax = qmode == ORC_FP8E4M3_B32 ? E4M3_MAX : qmode == ORC_FP8E5M2_B32 ? E5M2_MAX : 127.0f;
            float scale = amax / qmax;
            ((float*)scales)[g] = scale;
            for (int i = 0; i < 32; ++i) {
                uint8_t c = 0x00;
                if (scale != 0.0f) {
                    float y = xg[i] / scale;
                    if (qmode == ORC_FP8E4M3_B32) c = orc_e4m3fn_encode(y);
                    else if (qmode == ORC_FP8E5M2_B32) c = orc_e5m2_encode(y);
                    else {
                        float r = rintf(y);
                        if (r > 127.0f) r = 127.0f;
                        if (r < -127.0f) r = -127.0f;
                        c = (uint8_t)(int8_t)(int)r;
                    }
                }
                codes[32 * g + i] = c;
            }
        } else {
            /* MX: E8M0 power-of-two scale X, codes of x / X (exact division) */
            int e1m2 = qmode == ORC_MXFP4E1M2_B32;
            int fp4 = qmode == ORC_MXFP4_B32 || e1m2;
            float qmax = e1m2 ? E1M2_MAX : fp4 ? E2M1_MAX : E4M3_MAX;
            int emax = e1m2 ? 1 : fp4 ? 2 : 8;
            uint8_t e8 = (flags & ORC_MX_SCALE_OCP) ? orc_e8m0_floor(amax, emax)
                                                    : orc_e8m0_ceil(amax / qmax);
            float X = orc_e8m0_value(e8);
            ((uint8_t*)scales)[g] = e8;
            if (fp4) {
                for (int i = 0; i < 16; ++i) {
                    float y0 = xg[2 * i] / X, y1 = xg[2 * i + 1] / X;
                    uint8_t c0 = e1m2 ? orc_e1m2_encode(y0) : orc_e2m1_encode(y0);
                    uint8_t c1 = e1m2 ? orc_e1m2_encode(y1) : orc_e2m1_encode(y1);
                    codes[16 * g + i] = (uint8_t)(c0 | (c1 << 4));
                }
            } else {
                for (int i = 0; i < 32; ++i) codes[32 * g + i] = orc_e4m3fn_encode(xg[i] / X);
            }
        }
    }
}

/* Dequantized value of element d of one cache row, exact in fp64. */
static double dequant_elem(int qmode, const uint8_t* codes, const void* scales,
                           int zp, int d) {
    switch (qmode) {
    case ORC_INT8_TH:
        return ((double)(int8_t)codes[d] - zp) * (double)((const float*)scales)[0];
    case ORC_UINT4_TH: {
        int c = (codes[d / 2] >> (4 * (d & 1))) & 0xF;
        return ((double)c - zp) * (double)((const float*)scales)[0];
    }
    case ORC_FP8E4M3_B32:
        return (double)orc_e4m3fn_decode(codes[d]) * (double)((const float*)scales)[d / 32];
    case ORC_MXFP8_B32:
        return (double)orc_e4m3fn_decode(codes[d]) *
               (double)orc_e8m0_value(((const uint8_t*)scales)[d / 32]);
    case ORC_FP8E5M2_B32:
        return (double)orc_e5m2_decode(codes[d]) * (double)((const float*)scales)[d / 32];
    case ORC_INT8_B32:
        return (double)(int8_t)codes[d] * (double)((const float*)scales)[d / 32];
    case ORC_MXFP4E1M2_B32: {
        int c = (codes[d / 2] >> (4 * (d & 1))) & 0xF;
        return (double)orc_e1m2_decode((uint8_t)c) *
               (double)orc_e8m0_value(((const uint8_t*)scales)[d / 32]);
    }
    default: {
        int c = (codes[d / 2] >> (4 * (d & 1))) & 0xF;
        return (double)orc_e2m1_decode((uint8_t)c) *
               (double)orc_e8m0_value(((const uint8_t*)scales)[d / 32]);
    }
    }
}

/* Cache plane addressing: codes [B,H,S,row_bytes], scales [B,H,S,spr]
 * (float, or uint8 for MX-FP4), zps [B,H,S] (int8, affine modes only). */
static size_t cache_row(int H, int S, int b, int h, int s) {
    return ((size_t)b * H + h) * (size_t)S + (size_t)s;
}

static void* scale_ptr(int qmode, void* scales, size_t row, int spr) {
    if (e8m0_scales(qmode)) return (uint8_t*)scales + row * spr;
    return (float*)scales + row * spr;
}

/* Quantize a row of one cache in place; exposed for the pin tests. */
void orc_quantize_rows_f(int qmode, int flags, const float* x, int n_rows, int D,
                         uint8_t* codes, void* scales, int8_t* zps) {
    int rb = row_bytes(qmode, D), spr = scales_per_row(qmode, D);
    for (int r = 0; r < n_rows; ++r) {
        int8_t zp = 0;
        quantize_row(qmode, flags, x + (size_t)r * D, D, codes + (size_t)r * rb,
                     scale_ptr(qmode, scales, (size_t)r, spr), &zp);
        if (zps) zps[r] = zp;
    }
}
void orc_quantize_rows(int qmode, const float* x, int n_rows, int D,
                       uint8_t* codes, void* scales, int8_t* zps) {
    orc_quantize_rows_f(qmode, 0, x, n_rows, D, codes, scales, zps);
}

void orc_dequantize_rows(int qmode, const uint8_t* codes, const void* scales,
                         const int8_t* zps, int n_rows, int D, double* out) {
    int rb = row_bytes(qmode, D), spr = scales_per_row(qmode, D);
    for (int r = 0; r < n_rows; ++r)
        for (int d = 0; d < D; ++d)
            out[(size_t)r * D + d] = dequant_elem(
                qmode, codes + (size_t)r * rb,
                scale_ptr(qmode, (void*)scales, (size_t)r, spr),
                zps ? zps[r] : 0, d);
}

/* ------------------------------------------------------------------------ */
/* O5: quantize + scatter by slot ([IQC] parameter table and constraints;    */
/* [PR24473] update_cache_with_indices; [PR20351] static index_copy_)        */
/* ------------------------------------------------------------------------ */

/* x is [B, H, T, D] fp32 (bf16 inputs widened exactly), contiguous.
 * slot_mapping[b * slot_stride_b + t]; -1 skips the token, any other value
 * outside [0, n_slots) skips it and raises ORC_FLAG_SLOT_RANGE.  Every head
 * of token (b, t) is written to row (b, h, slot).  Returns the flags. */
int orc_quant_scatter_f(int qmode, int qflags, const float* x, int B, int H, int T, int D,
                        const int32_t* slot_mapping, long long slot_stride_b,
                        int n_slots, uint8_t* codes, void* scales, int8_t* zps) {
    int flags = 0;
    int rb = row_bytes(qmode, D), spr = scales_per_row(qmode, D);
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < T; ++t) {
            int32_t s = slot_mapping[(long long)b * slot_stride_b + t];
            if (s == -1) continue;
            if (s < -1 || s >= n_slots) { flags |= ORC_FLAG_SLOT_RANGE; continue; }
            for (int h = 0; h < H; ++h) {
                size_t row = cache_row(H, n_slots, b, h, s);
                int8_t zp = 0;
                quantize_row(qmode, qflags, x + (((size_t)b * H + h) * T + t) * D, D,
                             codes + row * rb, scale_ptr(qmode, scales, row, spr), &zp);
                if (qmode == ORC_INT8_TH || qmode == ORC_UINT4_TH) zps[row] = zp;
            }
        }
    return flags;
}
int orc_quant_scatter(int qmode, const float* x, int B, int H, int T, int D,
                      const int32_t* slot_mapping, long long slot_stride_b,
                      int n_slots, uint8_t* codes, void* scales, int8_t* zps) {
    return orc_quant_scatter_f(qmode, 0, x, B, H, T, D, slot_mapping, slot_stride_b, n_slots, codes, scales, zps);
}

/* ------------------------------------------------------------------------ */
/* O6: slot positions ([PR24473] Summary: sink = pinned prefix then a ring;   */
/* ring = sink with sink_size 0; full context = slot is the position)        */
/* ------------------------------------------------------------------------ */

/* Sink/ring layout: positions start_pos .. start_pos+T-1 in increasing
 * order, n_slots = sink + window, slot = p (p < sink) else
 * sink + (p - sink) mod window.  cache_positions (may be NULL) receives
 * cache_positions[slot] = p, so a later position wins its slot. */
int orc_positions_sink(int start_pos, int T, int sink, int window,
                       int32_t* slot_mapping, int32_t* cache_positions) {
    for (int t = 0; t < T; ++t) {
        int p = start_pos + t;
        int slot = p < sink ? p : sink + (p - sink) % window;
        slot_mapping[t] = slot;
        if (cache_positions) cache_positions[slot] = p;
    }
    /* R25: tokens are written one after another, so a token whose slot a
     * later token of the same call takes again leaves nothing behind; it gets
     * slot -1 (found by a backward scan over the slots already claimed). */
    int S = sink + window;
    unsigned char* taken = (unsigned char*)calloc((size_t)S, 1);
    for (int t = T - 1; t >= 0; --t) {
        int slot = slot_mapping[t];
        if (taken[slot]) slot_mapping[t] = -1;
        else taken[slot] = 1;
    }
    free(taken);
    return 0;
}

/* Full-context layout: slot = p; a position past the capacity is rejected
 * (slot -1, ORC_FLAG_POS_CAPACITY) instead of being written. */
int orc_positions_full(int start_pos, int T, int capacity,
                       int32_t* slot_mapping, int32_t* cache_positions) {
    int flags = 0;
    for (int t = 0; t < T; ++t) {
        int p = start_pos + t;
        if (p >= capacity) { slot_mapping[t] = -1; flags |= ORC_FLAG_POS_CAPACITY; continue; }
        slot_mapping[t] = p;
        if (cache_positions) cache_positions[p] = p;
    }
    return flags;
}

/* ------------------------------------------------------------------------ */
/* O7: additive mask for ring/sink caches ([PR24473] Summary; reading R11)   */
/* ------------------------------------------------------------------------ */

void orc_build_mask(const int32_t* cache_positions, int n_slots, int p0, int Lq,
                    int sink, int window, float* mask) {
    for (int r = 0; r < Lq; ++r) {
        int qp = p0 + r;
        for (int s = 0; s < n_slots; ++s) {
            int cp = cache_positions[s];
            int visible = cp >= 0 && cp <= qp && (cp < sink || qp - cp < window);
            mask[(size_t)r * n_slots + s] = visible ? 0.0f : -INFINITY;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* O8: attention on the quantized cache, fp64 after exact dequantization     */
/* ([ABADDON] forward_attention; [PR20351] kv_len and causal bounds;         */
/* [PR24473] mask for ring/sink, plain causal for full context)              */
/* ------------------------------------------------------------------------ */

typedef struct {
    int qmode, B, H, S, D;
    const uint8_t* codes;
    const void* scales;
    const int8_t* zps;
} orc_cache_view;

/* One output row: batch b, query head h, query row r of Lq.
 * q is [B, Hq, Lq, D] fp64.  Key j in [0, kv_len) is allowed iff
 * (!causal || j <= kv_len - Lq + r) and mask (if any) is not -inf at
 * [b][r][j].  s_j = sm_scale * q.k_j + mask; o = softmax(s) . v. */
static void sdpa_row(const double* q, int Hq, int Lq, const orc_cache_view* K,
                     const orc_cache_view* V, int kv_len, const float* mask,
                     long long mask_stride_b, int causal, double sm_scale,
                     int b, int h, int r, double* out, double* scores) {
    int D = K->D;
    int group = Hq / K->H;
    int g = h / group;                                        /* R14 */
    const double* qr = q + (((size_t)b * Hq + h) * Lq + r) * D;
    int rbk = row_bytes(K->qmode, D), sprk = scales_per_row(K->qmode, D);
    int rbv = row_bytes(V->qmode, D), sprv = scales_per_row(V->qmode, D);
    double m = -INFINITY;
    for (int j = 0; j < kv_len; ++j) {
        double add = mask ? (double)mask[(long long)b * mask_stride_b + (size_t)r * K->S + j] : 0.0;
        int allowed = (!causal || j <= kv_len - Lq + r) && add != -INFINITY;
        if (!allowed) { scores[j] = -INFINITY; continue; }
        size_t row = cache_row(K->H, K->S, b, g, j);
        const uint8_t* kc = K->codes + row * rbk;
        const void* ks = scale_ptr(K->qmode, (void*)K->scales, row, sprk);
        int kzp = K->zps ? K->zps[row] : 0;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += qr[d] * dequant_elem(K->qmode, kc, ks, kzp, d);
        scores[j] = sm_scale * dot + add;
        if (scores[j] > m) m = scores[j];
    }
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    if (m == -INFINITY) return;                               /* R13 */
    double l = 0.0;
    for (int j = 0; j < kv_len; ++j) {
        if (scores[j] == -INFINITY) continue;
        double p = exp(scores[j] - m);
        l += p;
        size_t row = cache_row(V->H, V->S, b, g, j);
        const uint8_t* vc = V->codes + row * rbv;
        const void* vs = scale_ptr(V->qmode, (void*)V->scales, row, sprv);
        int vzp = V->zps ? V->zps[row] : 0;
        for (int d = 0; d < D; ++d) out[d] += p * dequant_elem(V->qmode, vc, vs, vzp, d);
    }
    for (int d = 0; d < D; ++d) out[d] /= l;
}

/* Full attention: out is [B, Hq, Lq, D] fp64.  kv_len <= 0 means the whole
 * cache (S).  Returns ORC_FLAG_KVLEN (and computes nothing) when kv_len is
 * outside [Lq, S]. */
int orc_sdpa(const double* q, int B, int Hq, int Lq,
             int qmode, int Hkv, int S, int D,
             const uint8_t* kcodes, const void* kscales, const int8_t* kzps,
             const uint8_t* vcodes, const void* vscales, const int8_t* vzps,
             int kv_len, const float* mask, long long mask_stride_b, int causal,
             double sm_scale, double* out) {
    if (kv_len <= 0) kv_len = S;
    if (kv_len < Lq || kv_len > S) return ORC_FLAG_KVLEN;
    orc_cache_view K = {qmode, B, Hkv, S, D, kcodes, kscales, kzps};
    orc_cache_view V = {qmode, B, Hkv, S, D, vcodes, vscales, vzps};
    long long n = (long long)B * Hq * Lq;
    #pragma omp parallel
    {
        double* scores = (double*)malloc(sizeof(double) * (size_t)kv_len);
        #pragma omp for schedule(dynamic, 1)
        for (long long i = 0; i < n; ++i) {
            int r = (int)(i % Lq);
            int h = (int)((i / Lq) % Hq);
            int b = (int)(i / ((long long)Lq * Hq));
            sdpa_row(q, Hq, Lq, &K, &V, kv_len, mask, mask_stride_b, causal,
                     sm_scale, b, h, r, out + (size_t)i * D, scores);
        }
        free(scores);
    }
    return 0;
}

/* Selected rows only: rows is [n_rows, 3] = (b, h, r); out is [n_rows, D]. */
int orc_sdpa_rows(const double* q, int B, int Hq, int Lq,
                  int qmode, int Hkv, int S, int D,
                  const uint8_t* kcodes, const void* kscales, const int8_t* kzps,
                  const uint8_t* vcodes, const void* vscales, const int8_t* vzps,
                  int kv_len, const float* mask, long long mask_stride_b, int causal,
                  double sm_scale, const int32_t* rows, int n_rows, double* out) {
    if (kv_len <= 0) kv_len = S;
    if (kv_len < Lq || kv_len > S) return ORC_FLAG_KVLEN;
    orc_cache_view K = {qmode, B, Hkv, S, D, kcodes, kscales, kzps};
    orc_cache_view V = {qmode, B, Hkv, S, D, vcodes, vscales, vzps};
    #pragma omp parallel
    {
        double* scores = (double*)malloc(sizeof(double) * (size_t)kv_len);
        #pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < n_rows; ++i)
            sdpa_row(q, Hq, Lq, &K, &V, kv_len, mask, mask_stride_b, causal, sm_scale,
                     rows[3 * i], rows[3 * i + 1], rows[3 * i + 2],
                     out + (size_t)i * D, scores);
        free(scores);
    }
    return 0;
}

/* Vector helpers for the pin tests: encode/decode arrays element by element. */
void orc_e4m3fn_encode_array(const float* y, uint8_t* out, long long n) {
    for (long long i = 0; i < n; ++i) out[i] = orc_e4m3fn_encode(y[i]);
}
void orc_e1m2_encode_array(const float* y, uint8_t* out, long long n) {
    for (long long i = 0; i < n; ++i) out[i] = orc_e1m2_encode(y[i]);
}

void orc_e2m1_encode_array(const float* y, uint8_t* out, long long n) {
    for (long long i = 0; i < n; ++i) out[i] = orc_e2m1_encode(y[i]);
}
void orc_e8m0_ceil_array(const float* s, uint8_t* out, long long n) {
    for (long long i = 0; i < n; ++i) out[i] = orc_e8m0_ceil(s[i]);
}

/* Quantize-scatter in parallel over batches for large caches: the same
 * arithmetic as orc_quant_scatter, rows split over threads.  Used to build
 * long histories (the arithmetic is per row, so the order does not matter). */
int orc_quant_scatter_par_f(int qmode, int qflags, const float* x, int B, int H, int T, int D,
                            const int32_t* slot_mapping, long long slot_stride_b,
                            int n_slots, uint8_t* codes, void* scales, int8_t* zps) {
    int flags = 0;
    int rb = row_bytes(qmode, D), spr = scales_per_row(qmode, D);
    long long n = (long long)B * H * T;
    #pragma omp parallel for schedule(static) reduction(|:flags)
    for (long long i = 0; i < n; ++i) {
        int t = (int)(i % T);
        int h = (int)((i / T) % H);
        int b = (int)(i / ((long long)T * H));
        int32_t s = slot_mapping[(long long)b * slot_stride_b + t];
        if (s == -1) continue;
        if (s < -1 || s >= n_slots) { flags |= ORC_FLAG_SLOT_RANGE; continue; }
        size_t row = cache_row(H, n_slots, b, h, s);
        int8_t zp = 0;
        quantize_row(qmode, qflags, x + (size_t)i * D, D, codes + row * rb,
                     scale_ptr(qmode, scales, row, spr), &zp);
        if (qmode == ORC_INT8_TH || qmode == ORC_UINT4_TH) zps[row] = zp;
    }
    return flags;
}

int orc_quant_scatter_par(int qmode, const float* x, int B, int H, int T, int D,
                          const int32_t* slot_mapping, long long slot_stride_b,
                          int n_slots, uint8_t* codes, void* scales, int8_t* zps) {
    return orc_quant_scatter_par_f(qmode, 0, x, B, H, T, D, slot_mapping, slot_stride_b, n_slots, codes, scales, zps);
}

void orc_e5m2_encode_array(const float* y, uint8_t* out, long long n) {
    for (long long i = 0; i < n; ++i) out[i] = orc_e5m2_encode(y[i]);
}
void orc_e8m0_floor_array(const float* a, int emax, uint8_t* out, long long n) {
    for (long long i = 0; i < n; ++i) out[i] = orc_e8m0_floor(a[i], emax);
}
