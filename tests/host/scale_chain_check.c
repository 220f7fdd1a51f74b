/* Exhaustive check of the division-free NVFP4 scale chain used by the GPU
 * quantizers against plain IEEE division, over every pair of BF16 maxima
 * (block maximum amax <= outer maximum A, both non-negative finite BF16):
 *   p  = RN(amax / 6)      via q = amax*R6, r = fma(-q, 6, amax), fma(r, R6, q)
 *   s  = RN(A / 2688)      the same with R2688 = RN(1/2688)
 *   sc = RN(p / s)         q = p*rs, r = fma(-q, s, p), fma(r, rs, q), rs = RN(1/s)
 * (sc = 0 when s = 0; quotients by s < 2^-64 take a true division in the
 * kernels and are skipped here).  sc only matters through its E4M3 code,
 * which is 0 for every sc <= 2^-10; below 2^-11 the residual of the
 * correction can underflow (subnormal p), so only differences where either
 * value exceeds 2^-11 are counted.  Prints the numbers of mismatches. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf(uint32_t h) { uint32_t u = h << 16; float f; memcpy(&f, &u, 4); return f; }

static float mk(float a, float b, float rb)
{
    float q = a * rb;
    float r = fmaf(-q, b, a);
    return fmaf(r, rb, q);
}

int main(void)
{
    volatile float one = 1.0f, six = 6.0f, c2688 = 2688.0f;
    const float R6 = one / six, R2688 = one / c2688;
    long long bad_p = 0, bad_s = 0, bad_sc = 0;
    for (uint32_t h = 0; h < 0x7F80; ++h) {   /* p and s: single-argument checks */
        float a = bf(h);
        if (mk(a, 6.0f, R6) != a / 6.0f) ++bad_p;
        if (mk(a, 2688.0f, R2688) != a / 2688.0f) ++bad_s;
    }
#pragma omp parallel for reduction(+ : bad_sc) schedule(dynamic, 64)
    for (int hA = 0; hA < 0x7F80; ++hA) {
        float A = bf((uint32_t)hA);
        float s = A / 2688.0f;
        if (s == 0.0f || s < 0x1p-64f) continue;
        volatile float vs = s;
        float rs = 1.0f / vs;
        for (uint32_t h = 0; h <= (uint32_t)hA; ++h) {
            float p = bf(h) / 6.0f;
            float ref = p / s;
            float got = mk(p, s, rs);
            if (got != ref && (ref > 0x1p-11f || got > 0x1p-11f)) ++bad_sc;
        }
    }
    printf("%lld %lld %lld\n", bad_p, bad_s, bad_sc);
    return (bad_p || bad_s || bad_sc) ? 1 : 0;
}
