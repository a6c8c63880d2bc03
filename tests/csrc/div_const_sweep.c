/* div_const_sweep.c -- exhaustive check behind the affine scatter's scale:
 * for n = 255 and n = 15 (qmax - qmin of the int8 and 4-bit affine modes),
 * s0 = RN(x * RN(1/n)), s1 = RN(s0 + RN(x - s0 * n) * RN(1/n)) (both steps
 * fused multiply-adds) equals the correctly rounded quotient RN(x / n) for
 * every finite float x >= 0.  Prints the number of mismatches per n and exits
 * non-zero if there is any.  Built and run by tests/test_div_const_sweep.py. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static uint64_t mismatches(float n) {
    const float c = 1.0f / n;
    uint64_t bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
    for (int64_t hi = 0; hi < 0x7f80; ++hi) {
        for (uint32_t lo = 0; lo < 0x10000u; ++lo) {
            const uint32_t u = ((uint32_t)hi << 16) | lo;
            float x;
            memcpy(&x, &u, 4);
            const float q = x / n;
            const float s0 = x * c;
            const float s1 = fmaf(fmaf(-s0, n, x), c, s0);
            if (memcmp(&q, &s1, 4) != 0) ++bad;
        }
    }
    return bad;
}

int main(void) {
    const float ns[2] = {255.0f, 15.0f};
    int rc = 0;
    for (int k = 0; k < 2; ++k) {
        const uint64_t bad = mismatches(ns[k]);
        printf("n=%g mismatches=%llu\n", ns[k], (unsigned long long)bad);
        if (bad) rc = 1;
    }
    return rc;
}
