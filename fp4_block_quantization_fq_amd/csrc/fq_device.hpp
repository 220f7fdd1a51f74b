// fq_device.hpp -- device-side building blocks of the FP4 quantizers (gfx950).
//
// Every function here reproduces one step of the format definitions bit for
// bit (IEEE binary32, round to nearest even, denormals kept):
//  - MXFP4 (OCP Microscaling Formats v1.0): E2M1 elements, E8M0 block scale
//    2^(floor(log2 amax) - 2), code clamped to 0..254.
//  - NVFP4: E4M3 block scale (OCP OFP8 v1.0) under an FP32 outer scale
//    amax / (6 * 448) -- per tensor, or per 128-element outer block as in
//    "Resumo Tecnico: TetraJet-v2", sec. 2.A.
//  - Stochastic rounding with E[round(x)] = x (TetraJet-v2, sec. 2.A), drawn
//    from Philox4x32-10 (Salmon et al., SC'11) keyed by seed and indexed by
//    element.
// The kernels are compiled with -ffp-contract=off: every float expression
// below is exactly the operation written.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fqdev {

enum { FMT_MX = 0, FMT_NVT = 1, FMT_NV128 = 2 };
enum { RND_RNE = 0, RND_SR = 1 };

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }

// Packed 16-bit unsigned max (v_pk_max_u16): per half-word maximum.
__device__ __forceinline__ uint32_t pkmax_u16(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t,
        __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}

// BF16 magnitudes order like their bit patterns once the sign is cleared, so
// the block maximum is an integer maximum over (bits & 0x7FFF).
__device__ __forceinline__ uint32_t absmax_bits_8(const uint4 &v)
{
    const uint32_t M = 0x7FFF7FFFu;
    uint32_t m = pkmax_u16(pkmax_u16(v.x & M, v.y & M), pkmax_u16(v.z & M, v.w & M));
    return max(m & 0xFFFFu, m >> 16);
}

// ---- cross-lane maximum with DPP (no LDS traffic) -------------------------
// quad_perm [1,0,3,2]: partner lane i^1
__device__ __forceinline__ uint32_t dpp_max_xor1(uint32_t v)
{
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
}
// quad_perm [2,3,0,1]: partner lane i^2
__device__ __forceinline__ uint32_t dpp_max_xor2(uint32_t v)
{
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
}
// row_half_mirror: lane i <-> 7-i within each group of 8 lanes
__device__ __forceinline__ uint32_t dpp_max_half_mirror(uint32_t v)
{
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
}
// row_ror:4 and row_ror:8 rotate within each row of 16 lanes
__device__ __forceinline__ uint32_t dpp_max_ror4(uint32_t v)
{
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t dpp_max_ror8(uint32_t v)
{
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));
}

// ---- E8M0 (MXFP4) ----------------------------------------------------------
// Scale code from the BF16 magnitude bits of the block maximum: the BF16
// exponent field is floor(log2 amax) + 127 for normal values; subnormal and
// zero maxima (field 0) fall below the clamp at 2^-127 anyway.
__device__ __forceinline__ uint32_t mx_scale_code(uint32_t amax_bits16)
{
    int e = (int)(amax_bits16 >> 7);      // BF16 exponent field
    return (uint32_t)max(e - 2, 0);       // clamp(floor(log2) - 2, -127, .) + 127
}
// 2^(code-127) and its exact reciprocal 2^(127-code) (code <= 252 here).
__device__ __forceinline__ float e8m0_value(uint32_t code)
{
    return code ? as_f(code << 23) : as_f(0x00400000u);
}
__device__ __forceinline__ float e8m0_recip(uint32_t code)
{
    return as_f((254u - code) << 23);
}

// ---- E4M3 (NVFP4 block scale) ----------------------------------------------
// Non-negative finite v -> E4M3 code, nearest even, saturating at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_encode_sat(float v)
{
    if (!(v < 448.0f)) return 0x7Eu;
    if (v < 0.015625f) {                  // below 2^-6: subnormal quantum 2^-9
        return (uint32_t)__builtin_rintf(v * 512.0f);   // exact scaling, RNE
    }
    uint32_t u = as_u(v);
    u += 0x7FFFFu + ((u >> 20) & 1u);     // round mantissa to 3 bits, ties even
    return (u >> 20) - 960u;              // rebias 127 -> 7 ((127-7) << 3 = 960)
}
__device__ __forceinline__ float e4m3_value(uint32_t code)
{
    return code >= 8u ? as_f((code + 960u) << 20) : (float)code * 0.001953125f;
}

// ---- correctly rounded quotient |x| / s ------------------------------------
// With rcp = RN(1/s) (a correctly rounded division, once per block), the
// sequence q = RN(ax * rcp); r = ax - q * s (exact by FMA); q' = RN(q + r * rcp)
// returns RN(ax / s) for every BF16 ax when the quotient and the residual are
// in the normal range (Markstein's correction step; verified exhaustively for
// all 2^7 BF16 significands against all 2^23 FP32 divisor significands).
// Callers keep s >= 2^-64 by rescaling both operands by 2^64 (exact) when the
// block scale is smaller; quotients below 2^-17 only ever map to code 0.
__device__ __forceinline__ float quot_rn(float ax, float s, float rcp)
{
    float q = ax * rcp;
    float r = __builtin_fmaf(-q, s, ax);
    return __builtin_fmaf(r, rcp, q);
}

// ---- E2M1 encoders ---------------------------------------------------------
// In [0,2) the grid step is 0.5, in [2,4) it is 1, in [4,8) it is 2.  Adding
// 2^22, 2^23 or 2^24 rounds a to that step with the FPU's round-to-nearest-
// even, and the even multiple is exactly the even E2M1 code.  e is the FP32
// exponent field of a clamped to [127, 130], so the step is 2^(e-128).
// Outputs: m (3-bit magnitude code) and g (its value, at most 6).
__device__ __forceinline__ void e2m1_rne(float a, uint32_t &m, float &g)
{
    uint32_t e = min(max(as_u(a) >> 23, 127u), 130u);
    uint32_t Mb = (e << 23) + (22u << 23);        // 2^(e-105)
    float t = a + as_f(Mb);                       // RNE to the grid step
    uint32_t steps = as_u(t) - Mb;                // multiples of the step
    m = min(steps + 2u * e - 254u, 7u);           // + 0/2/4 per binade
    g = __builtin_fminf(t - as_f(Mb), 6.0f);
}

// Stochastic rounding with a 16-bit draw r: N = floor(a * 2^16 / step) holds
// the grid index above the binade base in its upper half and the threshold
// T = floor(frac * 2^16) in its lower 16 bits; round up iff r < T.
__device__ __forceinline__ uint32_t e2m1_sr(float a, uint32_t r)
{
    uint32_t e = min(max(as_u(a) >> 23, 127u), 130u);
    float sc = as_f((271u - e) << 23);            // 2^(144-e) = 2^16 / step
    uint32_t N = (uint32_t)(a * sc);              // exact product, truncation
    uint32_t down = (N >> 16) + 2u * e - 254u;
    uint32_t up = (r < (N & 0xFFFFu)) ? 1u : 0u;
    return min(down + up, 7u);
}

// E2M1 magnitude code -> value (0, .5, 1, 1.5, 2, 3, 4, 6).
__device__ __forceinline__ float e2m1_value(uint32_t m)
{
    // m >= 2: exponent 126 + (m >> 1), mantissa bit m & 1  ==  (m + 252) << 22
    float big = as_f((m + 252u) << 22);
    return m >= 2u ? big : (m ? 0.5f : 0.0f);
}

// ---- Philox4x32-10 ---------------------------------------------------------
struct u32x4 { uint32_t v[4]; };

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    u32x4 o;
    o.v[0] = c0; o.v[1] = c1; o.v[2] = c2; o.v[3] = c3;
    return o;
}

// ---- BF16 helpers ----------------------------------------------------------
__device__ __forceinline__ uint32_t bf16_pair_rne(float lo, float hi)
{
    __bf16 a = (__bf16)lo, b = (__bf16)hi;        // v_cvt_pk_bf16_f32 (RNE)
    return (uint32_t)__builtin_bit_cast(unsigned short, a)
         | ((uint32_t)__builtin_bit_cast(unsigned short, b) << 16);
}
// FP32 bits of element j (0..7) of a 16-byte BF16 vector.
__device__ __forceinline__ uint32_t elem_bits(const uint4 &v, int j)
{
    uint32_t w = (j >> 1) == 0 ? v.x : (j >> 1) == 1 ? v.y : (j >> 1) == 2 ? v.z : v.w;
    return (j & 1) ? (w & 0xFFFF0000u) : (w << 16);
}

// ---- per-block scale state ---------------------------------------------------
// s_eff: effective scale; rcp: RN(1/s_eff') and sq: s_eff' where s_eff' is
// s_eff rescaled by 2^64 when it is below 2^-64 (then xs = 2^64 scales |x|),
// so that the quotient sequence stays in the normal range.
struct BlockScale {
    float s_eff;
    float sq;
    float rcp;
    float xs;
    uint32_t code;
};

__device__ __forceinline__ BlockScale mx_block_scale(uint32_t amax_bits16)
{
    BlockScale b;
    b.code = mx_scale_code(amax_bits16);
    b.s_eff = e8m0_value(b.code);
    b.rcp = e8m0_recip(b.code);
    b.sq = b.s_eff;
    b.xs = 1.0f;
    return b;
}

// Quotient set-up for an NVFP4 block of effective scale s_eff.  A zero scale
// (the E4M3 code or its product with the outer scale underflowed) maps every
// element to a = 0: xs = 0 zeroes |x| before the quotient.  Scales below
// 2^-64 are rescaled with |x| by 2^64; the block's elements are then at most
// about 9 * s_eff, so the scaled |x| stays finite.
__device__ __forceinline__ void finish_nv_scale(BlockScale &b)
{
    b.xs = 1.0f;
    b.sq = b.s_eff;
    b.rcp = 0.0f;
    if (b.s_eff == 0.0f) {
        b.xs = 0.0f;
        b.sq = 1.0f;
        return;
    }
    if (b.s_eff < 0x1p-64f) {
        b.xs = 0x1p64f;
        b.sq = b.s_eff * 0x1p64f;
    }
    b.rcp = 1.0f / b.sq;
}

// NVFP4 block scale under outer scale s: e4 = E4M3(RN(RN(amax/6) / s)),
// s_eff = RN(e4 * s).
__device__ __forceinline__ BlockScale nv_block_scale(float amax, float s)
{
    BlockScale b;
    float sc = 0.0f;
    if (s != 0.0f) {
        float p = amax / 6.0f;
        sc = p / s;
    }
    b.code = e4m3_encode_sat(sc);
    b.s_eff = e4m3_value(b.code) * s;
    finish_nv_scale(b);
    return b;
}

// Scaled magnitude a = RN(|x| / s_eff) for the block.
template <int FMT>
__device__ __forceinline__ float scaled_mag(uint32_t xbits, const BlockScale &b)
{
    float ax = as_f(xbits & 0x7FFFFFFFu);
    if (FMT == FMT_MX) return ax * b.rcp;         // power-of-two scale: exact
    return quot_rn(ax * b.xs, b.sq, b.rcp);
}

// NVFP4 outer scale amax / (6 * 448).
__device__ __forceinline__ float nv_outer_scale(float amax)
{
    return amax / 2688.0f;
}

}  // namespace fqdev
