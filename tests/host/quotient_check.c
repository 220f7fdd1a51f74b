/* Exhaustive check of the division used by the GPU quantizers:
 *   rcp = RN(1/s); q = RN(x*rcp); r = fma(-q, s, x); q' = fma(r, rcp, q)
 * must equal RN(x/s) for every BF16 significand of x (2^7 values) and every
 * FP32 significand of s (2^23 values).  Exponents only shift the quotient, so
 * x, s in [1, 2) covers every normal-range case.  Prints the mismatch count. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_from(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

int main(void)
{
    long long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(dynamic, 1 << 16)
    for (long long j = 0; j < (1LL << 23); ++j) {
        float s = f_from(0x3F800000u | (uint32_t)j);
        volatile float one = 1.0f;
        float rcp = one / s;
        for (uint32_t i = 0; i < 128; ++i) {
            float x = f_from(0x3F800000u | (i << 16));
            float q = x * rcp;
            float r = fmaf(-q, s, x);
            float q2 = fmaf(r, rcp, q);
            float ref = x / s;
            if (q2 != ref) ++bad;
        }
    }
    printf("%lld\n", bad);
    return bad != 0;
}
