// encoder_sweep.hip -- the element encoders of the block quant-scatter
// (kvq_device.h: magnitude clamp + gfx950 conversion instruction) against
// bit-level round-to-nearest-even encoders written from the format
// definitions (FP8 E4M3FN: bias 7, 3 mantissa bits, largest 448, no inf;
// FP8 E5M2: bias 15, 2 mantissa bits, largest finite 57344; FP4 E2M1:
// magnitudes 0 .5 1 1.5 2 3 4 6), saturating at the largest value with the
// sign kept, over every one of the 2^32 fp32 bit patterns.
//
// Each thread covers 256 consecutive patterns (65536 x 256 threads); the
// mismatch count and the first 16 mismatches go to a small device buffer.
// Exit status 0 when all three formats match everywhere.
#include <hip/hip_runtime.h>
#include <cstdint>
#include <cstdio>

#include "../../quantized_kv_cache_head_amd/csrc/kvq_device.h"

using namespace kvq;

// FP8 E4M3FN, round to nearest even, |y| >= 448 saturates to 0x7E, sign kept.
__device__ __forceinline__ uint32_t ref_e4m3fn(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t mag;
    if (a >= 0x43E00000u) {                 // >= 448
        mag = 0x7Eu;
    } else if (a < 0x3C800000u) {           // < 2^-6: multiples of 2^-9
        mag = (uint32_t)rintf(__uint_as_float(a) * 512.0f);
    } else {                                // keep 3 mantissa bits, RNE
        const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
        mag = (r >> 20) - (120u << 3);      // rebias exponent 127 -> 7
    }
    return sign | mag;
}
// FP4 E2M1 (magnitudes 0,.5,1,1.5,2,3,4,6), RNE, |y| >= 6 saturates, sign bit 3.
__device__ __forceinline__ uint32_t ref_e2m1(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 28) & 0x8u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t mag;
    if (a >= 0x40C00000u) {                 // >= 6
        mag = 7u;
    } else if (a < 0x3F800000u) {           // < 1: multiples of 0.5
        mag = (uint32_t)rintf(__uint_as_float(a) * 2.0f);
    } else {                                // keep 1 mantissa bit, RNE
        const uint32_t r = a + 0x1FFFFFu + ((a >> 22) & 1u);
        mag = (r >> 22) - (126u << 1);      // rebias exponent 127 -> 1
    }
    return sign | mag;
}
// FP8 E5M2 (bias 15, 2 mantissa bits), round to nearest even, |y| >= 57344
// saturates to 0x7B (never inf), sign kept.
__device__ __forceinline__ uint32_t ref_e5m2(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t mag;
    if (a >= 0x47600000u) {                 // >= 57344
        mag = 0x7Bu;
    } else if (a < 0x38800000u) {           // < 2^-14: multiples of 2^-16
        mag = (uint32_t)rintf(__uint_as_float(a) * 65536.0f);
    } else {                                // keep 2 mantissa bits, RNE
        const uint32_t r = a + 0xFFFFFu + ((a >> 21) & 1u);
        mag = (r >> 21) - (112u << 2);      // rebias exponent 127 -> 15
    }
    return sign | mag;
}

template <int F>
__global__ void sweep(unsigned long long* bad, uint32_t* first) {
    const uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint32_t base = (uint32_t)(t * 256u);
    unsigned nb = 0;
    for (uint32_t i = 0; i < 256; i += 8) {
        float y[8];
        for (int e = 0; e < 8; ++e) y[e] = __uint_as_float(base + i + e);
        uint32_t hw[8], sw[8];
        if constexpr (F == 2) {
            const uint32_t w = cvt8_e2m1(y);
            for (int e = 0; e < 8; ++e) { hw[e] = (w >> (4 * e)) & 0xFu; sw[e] = ref_e2m1(y[e]); }
        } else {
            const uint32_t w0 = F == 0 ? cvt4_e4m3fn(y) : cvt4_e5m2(y);
            const uint32_t w1 = F == 0 ? cvt4_e4m3fn(y + 4) : cvt4_e5m2(y + 4);
            for (int e = 0; e < 8; ++e) {
                hw[e] = ((e < 4 ? w0 : w1) >> (8 * (e & 3))) & 0xFFu;
                sw[e] = F == 0 ? ref_e4m3fn(y[e]) : ref_e5m2(y[e]);
            }
        }
        for (int e = 0; e < 8; ++e) {
            if (hw[e] != sw[e]) {
                ++nb;
                const unsigned long long k = atomicAdd(bad + 1, 1ull);
                if (k < 16) {
                    first[3 * k] = base + i + e;
                    first[3 * k + 1] = hw[e];
                    first[3 * k + 2] = sw[e];
                }
            }
        }
    }
    if (nb) atomicAdd(bad, (unsigned long long)nb);
}

int main() {
    unsigned long long* bad = nullptr;
    uint32_t* first = nullptr;
    if (hipMalloc(&bad, 16) != hipSuccess || hipMalloc(&first, 48 * sizeof(uint32_t)) != hipSuccess) {
        printf("allocation failed\n");
        return 2;
    }
    const char* names[3] = {"e4m3fn", "e5m2", "e2m1"};
    const unsigned blocks = 65536;                   // 65536 x 256 threads x 256 patterns = 2^32
    int rc = 0;
    for (int f = 0; f < 3; ++f) {
        if (hipMemset(bad, 0, 16) != hipSuccess || hipMemset(first, 0, 48 * sizeof(uint32_t)) != hipSuccess) return 2;
        if (f == 0) hipLaunchKernelGGL(sweep<0>, dim3(blocks), dim3(256), 0, 0, bad, first);
        if (f == 1) hipLaunchKernelGGL(sweep<1>, dim3(blocks), dim3(256), 0, 0, bad, first);
        if (f == 2) hipLaunchKernelGGL(sweep<2>, dim3(blocks), dim3(256), 0, 0, bad, first);
        const hipError_t e = hipDeviceSynchronize();
        unsigned long long hb[2] = {0, 0};
        uint32_t hf[48] = {0};
        if (hipMemcpy(hb, bad, 16, hipMemcpyDeviceToHost) != hipSuccess ||
            hipMemcpy(hf, first, sizeof hf, hipMemcpyDeviceToHost) != hipSuccess)
            return 2;
        printf("%s: %s, mismatches %llu\n", names[f], hipGetErrorString(e), hb[0]);
        for (int k = 0; k < 16 && k < (int)hb[1]; ++k)
            printf("  y 0x%08x instruction %02x reference %02x\n", hf[3 * k], hf[3 * k + 1], hf[3 * k + 2]);
        if (hb[0] || e != hipSuccess) rc = 1;
    }
    return rc;
}
