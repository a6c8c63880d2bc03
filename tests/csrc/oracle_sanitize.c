/* Driver that runs every entry point of the CPU oracle on small, seeded
 * inputs (all seven cache modes, slot -1 and out-of-range slots, every
 * encoder on edge values, positions, masks, attention with mask / causal /
 * kv_len), built together with oracle/kvq_oracle.c under gcc's address and
 * undefined-behaviour sanitizers by tests/test_oracle_sanitize.py.  A
 * sanitizer report aborts the process; a clean run prints "oracle sanitize ok". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint8_t orc_e4m3fn_encode(float y);
float orc_e4m3fn_decode(uint8_t code);
uint8_t orc_e2m1_encode(float y);
float orc_e2m1_decode(uint8_t code);
uint8_t orc_e1m2_encode(float y);
float orc_e1m2_decode(uint8_t code);
uint8_t orc_e8m0_ceil(float s);
uint8_t orc_e8m0_floor(float amax, int emax);
uint8_t orc_e5m2_encode(float y);
float orc_e5m2_decode(uint8_t code);
int orc_row_bytes(int qmode, int D);
int orc_scales_per_row(int qmode, int D);
void orc_quantize_rows_f(int qmode, int flags, const float* x, int n_rows, int D, uint8_t* codes, void* scales,
                         int8_t* zps);
void orc_dequantize_rows(int qmode, const uint8_t* codes, const void* scales, const int8_t* zps, int n_rows, int D,
                         double* out);
int orc_quant_scatter_f(int qmode, int qflags, const float* x, int B, int H, int T, int D, const int32_t* slot_mapping,
                        long long slot_stride_b, int n_slots, uint8_t* codes, void* scales, int8_t* zps);
int orc_quant_scatter_par_f(int qmode, int qflags, const float* x, int B, int H, int T, int D,
                            const int32_t* slot_mapping, long long slot_stride_b, int n_slots, uint8_t* codes,
                            void* scales, int8_t* zps);
int orc_positions_sink(int start_pos, int T, int sink, int window, int32_t* slot_mapping, int32_t* cache_positions);
int orc_positions_full(int start_pos, int T, int capacity, int32_t* slot_mapping, int32_t* cache_positions);
void orc_build_mask(const int32_t* cache_positions, int n_slots, int p0, int Lq, int sink, int window, float* mask);
int orc_sdpa(const double* q, int B, int Hq, int Lq, int qmode, int Hkv, int S, int D, const uint8_t* kcodes,
             const void* kscales, const int8_t* kzps, const uint8_t* vcodes, const void* vscales, const int8_t* vzps,
             int kv_len, const float* mask, long long mask_stride_b, int causal, double sm_scale, double* out);
int orc_sdpa_rows(const double* q, int B, int Hq, int Lq, int qmode, int Hkv, int S, int D, const uint8_t* kcodes,
                  const void* kscales, const int8_t* kzps, const uint8_t* vcodes, const void* vscales,
                  const int8_t* vzps, int kv_len, const float* mask, long long mask_stride_b, int causal,
                  double sm_scale, const int32_t* rows, int n_rows, double* out);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double uniform(void) {   /* splitmix64 */
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) / 9007199254740992.0;
}
static float normal(void) {
    double u1 = uniform(), u2 = uniform();
    if (u1 < 1e-300) u1 = 1e-300;
    return (float)(sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
}

static int mx_mode(int qmode) { return qmode == 3 || qmode == 4 || qmode == 7; }
static size_t scale_bytes(int qmode) { return mx_mode(qmode) ? 1 : 4; }

int main(void) {
    /* encoders and decoders on edge values */
    const float edge[] = {0.0f, -0.0f, 1e-45f, -1e-45f, 1e-38f, 0.5f, 1.0f, 447.9f, 448.0f, 464.0f, 57344.0f,
                          1e30f, -1e30f, INFINITY, -INFINITY, NAN, 6.0f, 5.0f, 0.25f, 0.75f};
    unsigned acc = 0;
    for (size_t i = 0; i < sizeof(edge) / sizeof(edge[0]); ++i) {
        acc += orc_e4m3fn_encode(edge[i]) + orc_e2m1_encode(edge[i]) + orc_e5m2_encode(edge[i]) + orc_e1m2_encode(edge[i]);
        acc += orc_e8m0_ceil(fabsf(edge[i])) + orc_e8m0_floor(fabsf(edge[i]), 8) + orc_e8m0_floor(fabsf(edge[i]), 2);
        acc += orc_e8m0_floor(fabsf(edge[i]), 1);
    }
    for (int c = 0; c < 256; ++c) {
        volatile float f = orc_e4m3fn_decode((uint8_t)c) + orc_e5m2_decode((uint8_t)c);
        (void)f;
        if (c < 16) { volatile float g = orc_e2m1_decode((uint8_t)c) + orc_e1m2_decode((uint8_t)c); (void)g; }
    }
    /* quantize + scatter, every mode, both flags, serial and parallel */
    enum { B = 2, H = 3, T = 5, D = 64, S = 16, Hq = 6, Lq = 3 };
    float* x = malloc(sizeof(float) * B * H * T * D);
    for (int i = 0; i < B * H * T * D; ++i) x[i] = normal() * (i % 37 == 0 ? 20.0f : 1.0f);
    int32_t slots[B * T] = {0, 3, -1, 15, 7, 2, -1, 99, 4, -5};
    for (int qmode = 0; qmode <= 7; ++qmode) {
        const int rb = orc_row_bytes(qmode, D), spr = orc_scales_per_row(qmode, D);
        uint8_t* codes = calloc((size_t)B * H * S * rb, 1);
        void* scales = calloc((size_t)B * H * S * spr, scale_bytes(qmode));
        int8_t* zps = calloc((size_t)B * H * S, 1);
        for (int qflags = 0; qflags <= (mx_mode(qmode) ? 1 : 0); ++qflags) {
            int f1 = orc_quant_scatter_f(qmode, qflags, x, B, H, T, D, slots, T, S, codes, scales, zps);
            int f2 = orc_quant_scatter_par_f(qmode, qflags, x, B, H, T, D, slots, T, S, codes, scales, zps);
            if (f1 != 1 || f2 != 1) { printf("unexpected flags %d %d (mode %d)\n", f1, f2, qmode); return 1; }
        }
        double* deq = malloc(sizeof(double) * B * H * S * D);
        orc_dequantize_rows(qmode, codes, scales, zps, B * H * S, D, deq);
        /* attention over the cache: plain, causal, masked, selected rows */
        double* q = malloc(sizeof(double) * B * Hq * Lq * D);
        for (int i = 0; i < B * Hq * Lq * D; ++i) q[i] = normal();
        float* mask = malloc(sizeof(float) * B * Lq * S);
        for (int i = 0; i < B * Lq * S; ++i) mask[i] = (i % 5 == 1) ? -INFINITY : 0.0f;
        double* out = malloc(sizeof(double) * B * Hq * Lq * D);
        int r1 = orc_sdpa(q, B, Hq, Lq, qmode, H, S, D, codes, scales, zps, codes, scales, zps, 12, NULL, 0, 1, 0.125,
                          out);
        int r2 = orc_sdpa(q, B, Hq, Lq, qmode, H, S, D, codes, scales, zps, codes, scales, zps, 0, mask,
                          (long long)Lq * S, 0, 0.125, out);
        int r3 = orc_sdpa(q, B, Hq, Lq, qmode, H, S, D, codes, scales, zps, codes, scales, zps, 2, NULL, 0, 0, 0.125,
                          out);
        int32_t rows[6] = {0, 1, 2, 1, 5, 0};
        int r4 = orc_sdpa_rows(q, B, Hq, Lq, qmode, H, S, D, codes, scales, zps, codes, scales, zps, 9, mask,
                               (long long)Lq * S, 1, 0.125, rows, 2, out);
        if (r1 || r2 || r3 != 2 || r4) { printf("unexpected sdpa status %d %d %d %d\n", r1, r2, r3, r4); return 1; }
        free(codes); free(scales); free(zps); free(deq); free(q); free(mask); free(out);
    }
    /* rows of one quantize call, all modes, D 32 .. 256 */
    for (int qmode = 0; qmode <= 6; ++qmode)
        for (int d = 32; d <= 256; d *= 2) {
            uint8_t* codes = calloc((size_t)4 * orc_row_bytes(qmode, d), 1);
            void* scales = calloc((size_t)4 * orc_scales_per_row(qmode, d), scale_bytes(qmode));
            int8_t zps[4];
            float* xr = malloc(sizeof(float) * 4 * d);
            for (int i = 0; i < 4 * d; ++i) xr[i] = (i % 3 == 0) ? 0.0f : normal();
            for (int i = 0; i < d; ++i) xr[i] = 0.0f;   /* an all-zero row */
            orc_quantize_rows_f(qmode, 0, xr, 4, d, codes, scales, zps);
            free(codes); free(scales); free(xr);
        }
    /* positions and masks */
    int32_t sm[64], cp[68];
    for (int i = 0; i < 68; ++i) cp[i] = -1;
    for (int p = 0; p < 300; p += 7) orc_positions_sink(p, 5, 4, 64, sm, cp);
    orc_positions_sink(10, 64, 0, 68, sm, cp);
    int fl = orc_positions_full(60, 10, 64, sm, cp);
    if (fl != 4) { printf("unexpected full-context flags %d\n", fl); return 1; }
    float mk[3 * 68];
    orc_build_mask(cp, 68, 290, 3, 4, 64, mk);
    orc_build_mask(cp, 68, 0, 3, 0, 68, mk);
    free(x);
    printf("oracle sanitize ok (%u)\n", acc & 0xFF);
    return 0;
}
