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
//
// Work unit: one lane owns 16 consecutive elements along the quantization
// axis, held as 8 packed BF16 pairs.  That is one NVFP4 block, or half of an
// MXFP4 block (the partner lane is lane ^ 1).
//
// gfx950 conversion instructions used (their rounding was measured against
// the format definitions on every BF16 input and on FP32 inputs around every
// rounding threshold):
//  - v_cvt_scalef32_pk_fp4_{bf16,f32}: two values -> two E2M1 codes of
//    RNE(x / 2^floor(log2 scale)), sign kept, saturating at 6.  With a
//    power-of-two scale this is the MXFP4 encoder; with scale 1 it encodes a
//    precomputed NVFP4 quotient.
//  - v_cvt_scalef32_pk_{bf16,f32}_fp4: two codes -> +-g * 2^floor(log2 scale),
//    exact for power-of-two scales (code 8 gives -0.0).
// The kernels are compiled with -ffp-contract=off: every float expression
// below is exactly the operation written.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fqdev {

enum { FMT_MX = 0, FMT_NVT = 1, FMT_NV128 = 2 };
enum { RND_RNE = 0, RND_SR = 1 };

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

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
__device__ __forceinline__ uint32_t absmax_bits_pairs8(const uint32_t (&xp)[8])
{
    const uint32_t M = 0x7FFF7FFFu;
    uint32_t m01 = pkmax_u16(xp[0] & M, xp[1] & M), m23 = pkmax_u16(xp[2] & M, xp[3] & M);
    uint32_t m45 = pkmax_u16(xp[4] & M, xp[5] & M), m67 = pkmax_u16(xp[6] & M, xp[7] & M);
    uint32_t m = pkmax_u16(pkmax_u16(m01, m23), pkmax_u16(m45, m67));
    return max(m & 0xFFFFu, m >> 16);
}
__device__ __forceinline__ uint32_t absmax_bits_8(const uint4 &v)
{
    const uint32_t M = 0x7FFF7FFFu;
    uint32_t m = pkmax_u16(pkmax_u16(v.x & M, v.y & M), pkmax_u16(v.z & M, v.w & M));
    return max(m & 0xFFFFu, m >> 16);
}

// ---- cross-lane maximum with DPP (no LDS traffic) -------------------------
// Values are non-negative, so a disabled source lane (read as 0) is harmless.
__device__ __forceinline__ uint32_t dpp_max_xor1(uint32_t v)   // quad_perm [1,0,3,2]
{
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t dpp_max_xor2(uint32_t v)   // quad_perm [2,3,0,1]
{
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t dpp_max_half_mirror(uint32_t v)   // i <-> 7-i in 8 lanes
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
// maximum over the 8 lanes 8k..8k+7
__device__ __forceinline__ uint32_t dpp_max_8lanes(uint32_t v)
{
    return dpp_max_half_mirror(dpp_max_xor2(dpp_max_xor1(v)));
}

// ---- E8M0 (MXFP4) ----------------------------------------------------------
// Scale code from the BF16 magnitude bits of the block maximum: the BF16
// exponent field is floor(log2 amax) + 127 for normal values; subnormal and
// zero maxima (field 0) fall below the clamp at 2^-127 anyway.
__device__ __forceinline__ uint32_t mx_scale_code(uint32_t amax_bits16)
{
    return (uint32_t)max((int)(amax_bits16 >> 7) - 2, 0);
}
// 2^(code-127) (FP32 subnormal 2^-127 for code 0) and its exact reciprocal.
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

// ---- correctly rounded quotients -------------------------------------------
// q = RN(a * rb); r = a - q * b (exact by FMA); q' = RN(q + r * rb), with
// rb = RN(1/b).  This is RN(a / b):
//  - for every BF16 a and every FP32 b in the normal range (checked on the
//    host for all 2^7 x 2^23 significand pairs);
//  - for a = RN(amax / 6) and b = RN(A / 2688) with BF16 maxima amax <= A
//    and b >= 2^-64, wherever the result exceeds 2^-11 (checked for all pairs;
//    below that the E4M3 block scale is 0 either way).
__device__ __forceinline__ float div_corrected(float a, float b, float rb)
{
    float q = a * rb;
    float r = __builtin_fmaf(-q, b, a);
    return __builtin_fmaf(r, rb, q);
}
// Division of a BF16 value by 6 and by 2688 (checked for every BF16 input).
__device__ __forceinline__ float div6(float a) { return div_corrected(a, 6.0f, as_f(0x3E2AAAABu)); }
__device__ __forceinline__ float nv_outer_scale(float amax)
{
    return div_corrected(amax, 2688.0f, as_f(0x39C30C31u));
}

// ---- per-block scale state ---------------------------------------------------
// s_eff: effective scale; rcp: RN(1/sq) with sq = s_eff, or s_eff * 2^64 when
// s_eff < 2^-64 (then xs = 2^64 scales |x| too, keeping the quotient sequence
// in the normal range); a zero scale sets xs = 0 so every a is 0.
struct BlockScale {
    float s_eff;
    float sq;
    float rcp;
    float xs;
    uint32_t code;
};

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

// Outer scale s and its reciprocal rs = RN(1/s) (rs unused when s < 2^-64).
struct OuterScale {
    float s;
    float rs;
};
__device__ __forceinline__ OuterScale make_outer(float amax_outer)
{
    OuterScale o;
    o.s = nv_outer_scale(amax_outer);
    o.rs = (o.s >= 0x1p-64f) ? 1.0f / o.s : 0.0f;
    return o;
}

// NVFP4 block scale under outer scale s: e4 = E4M3(RN(RN(amax/6) / s)),
// s_eff = RN(e4 * s).
__device__ __forceinline__ BlockScale nv_block_scale(float amax, const OuterScale &o)
{
    BlockScale b;
    float sc = 0.0f;
    if (o.s != 0.0f) {
        const float p = div6(amax);
        sc = (o.s >= 0x1p-64f) ? div_corrected(p, o.s, o.rs) : p / o.s;
    }
    b.code = e4m3_encode_sat(sc);
    b.s_eff = e4m3_value(b.code) * o.s;
    finish_nv_scale(b);
    return b;
}

// Chunk mapping: lane owns 8 elements; an NVFP4 block is a lane pair, an
// MXFP4 block a lane quad and a 128-element outer block a DPP row of 16.
template <int FMT>
__device__ __forceinline__ BlockScale chunk_block_scale(uint32_t amax8, const OuterScale &ot,
                                                        float &outer_out)
{
    const uint32_t m = dpp_max_xor1(amax8);
    if (FMT == FMT_MX) return mx_block_scale(dpp_max_xor2(m));
    if (FMT == FMT_NVT) return nv_block_scale(as_f(m << 16), ot);
    const uint32_t mo = dpp_max_ror8(dpp_max_ror4(dpp_max_xor2(m)));
    const OuterScale o = make_outer(as_f(mo << 16));
    outer_out = o.s;
    return nv_block_scale(as_f(m << 16), o);
}

template <int FMT>
__device__ __forceinline__ BlockScale scale_from_code(uint32_t code, float s)
{
    BlockScale b;
    b.code = code;
    b.xs = 1.0f;
    if (FMT == FMT_MX) {
        b.s_eff = e8m0_value(code);
        b.rcp = e8m0_recip(code);
        b.sq = b.s_eff;
    } else {
        b.s_eff = e4m3_value(code) * s;
        finish_nv_scale(b);
    }
    return b;
}

// Scaled magnitude a = RN(|x| / s_eff) (x as FP32 bits).
template <int FMT>
__device__ __forceinline__ float scaled_mag(uint32_t xbits, const BlockScale &b)
{
    float ax = as_f(xbits & 0x7FFFFFFFu);
    if (FMT == FMT_MX) return ax * b.rcp;         // power-of-two scale: exact
    return div_corrected(ax * b.xs, b.sq, b.rcp);
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
        uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);  // xor3
        uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
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
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
__device__ __forceinline__ uint32_t lo_bits(uint32_t pair) { return pair << 16; }
__device__ __forceinline__ uint32_t hi_bits(uint32_t pair) { return pair & 0xFFFF0000u; }

// ---- random Hadamard transform of one 16-element segment ---------------------
// "Resumo Tecnico: TetraJet-v2", sec. 2.C (OutControl): blockwise H_n (n = 16
// or 128) with a Philox-seeded random sign vector, in Sylvester order by
// radix-2 FP32 butterflies, times the FP32 value nearest to 1/sqrt(n), rounded
// to BF16.  Sign bit of position j: bit (j mod 128) of Philox4x32-10(key =
// seed, counter = (j / 128, 0, 0, 0)), bit t of word w being bit 32w + t.
// The 16 sign bits of positions j0 .. j0 + 15 (j0 a multiple of 16).
__device__ __forceinline__ uint32_t sign_bits16(uint64_t j0, uint32_t seed_lo, uint32_t seed_hi)
{
    const u32x4 o = philox4x32_10((uint32_t)(j0 >> 7), (uint32_t)(j0 >> 39), 0u, 0u, seed_lo,
                                  seed_hi);
    const uint32_t b = (uint32_t)(j0 & 127);
    const uint32_t w = o.v[b >> 5];
    return (w >> (b & 31)) & 0xFFFFu;
}

// In-lane stages h = 1, 2, 4, 8 over 16 values.
__device__ __forceinline__ void fwht16(float (&v)[16])
{
#pragma unroll
    for (int h = 1; h < 16; h *= 2)
#pragma unroll
        for (int g = 0; g < 16; g += 2 * h)
#pragma unroll
            for (int t = g; t < g + h; ++t) {
                const float a = v[t], b = v[t + h];
                v[t] = a + b;
                v[t + h] = a - b;
            }
}

// The value of lane ^ D (D = 1, 2, 4) by DPP inside the lane's 16-lane row,
// with no LDS traffic: quad permutes for 1 and 2; for 4 a rotation of the row
// by 12 (lane + 4, lanes with bit 2 clear) or by 4 (lane - 4, bit 2 set).
template <int D>
__device__ __forceinline__ float lane_xor(float v, bool bit2)
{
    const int iv = __float_as_int(v);
    if (D == 1) return __int_as_float(__builtin_amdgcn_update_dpp(0, iv, 0xB1, 0xF, 0xF, false));
    if (D == 2) return __int_as_float(__builtin_amdgcn_update_dpp(0, iv, 0x4E, 0xF, 0xF, false));
    const int up = __builtin_amdgcn_update_dpp(0, iv, 0x12C, 0xF, 0xF, false);    // row_ror:12
    const int dn = __builtin_amdgcn_update_dpp(0, iv, 0x124, 0xF, 0xF, false);    // row_ror:4
    return __int_as_float(bit2 ? dn : up);
}

template <int D>
__device__ __forceinline__ void fwht_lane_stage(float (&v)[16], uint32_t lane_in_block)
{
    // lower lane of a pair: a + b; upper: b - a = b + (-a), with b the
    // partner's value (the same sums, exactly rounded, in either order)
    const uint32_t neg = (lane_in_block & D) ? 0x80000000u : 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float p = lane_xor<D>(v[i], (lane_in_block & 4) != 0);
        v[i] = p + as_f(as_u(v[i]) ^ neg);
    }
}

// Cross-lane stages for n = 128: lane offsets 1, 2, 4 (element half-widths
// 16, 32, 64).  The lower lane of a pair keeps a + b, the upper a - b, with a
// the lower lane's value.  The 8 lanes of a 128-block are 8 aligned lanes of
// the wave (lane_in_block = lane mod 8).
__device__ __forceinline__ void fwht_lanes(float (&v)[16], uint32_t lane_in_block)
{
    fwht_lane_stage<1>(v, lane_in_block);
    fwht_lane_stage<2>(v, lane_in_block);
    fwht_lane_stage<4>(v, lane_in_block);
}

__device__ __forceinline__ float flip(float e, uint32_t bits, int i)
{
    return as_f(as_u(e) ^ (((bits >> i) & 1u) << 31));
}

// Rotate the lane's segment in place: xp holds 16 consecutive positions
// j0 .. j0 + 15 along the transformed axis as BF16 pairs (position 2i in the
// low half of xp[i]); for n = 128 the 8 lanes of a 128-block are lanes
// 8k .. 8k + 7, lane_in_block = (j0 / 16) mod 8.
template <int N>
__device__ __forceinline__ void rht_segment(uint32_t (&xp)[8], uint64_t j0, uint32_t seed_lo,
                                            uint32_t seed_hi)
{
    const uint32_t bits = sign_bits16(j0, seed_lo, seed_hi);
    float v[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = flip(as_f(lo_bits(xp[i])), bits, 2 * i);
        v[2 * i + 1] = flip(as_f(hi_bits(xp[i])), bits, 2 * i + 1);
    }
    fwht16(v);
    if (N == 128) fwht_lanes(v, (uint32_t)(j0 >> 4) & 7);
    const float c_n = N == 16 ? 0.25f : __builtin_bit_cast(float, 0x3DB504F3u);
#pragma unroll
    for (int i = 0; i < 8; ++i) xp[i] = bf16_pair_rne(c_n * v[2 * i], c_n * v[2 * i + 1]);
}

// ---- column tile in LDS (column quantizer, column Hadamard transform) ------
// A 64-column x 256-row BF16 tile: LDS block b holds tile rows 8b .. 8b+7,
// 128 bytes each, and the 16-byte chunk of columns 8g .. 8g+7 of a row in
// block b sits in slot g ^ ((b >> 1) & 7), so that eight lanes reading one
// chunk of eight row blocks hit eight different slots.
typedef __attribute__((address_space(3))) void lds_void;   // direct-load LDS target
constexpr uint32_t kQcCols = 64, kQcRows = 256, kQcThreads = 512;
constexpr uint32_t kQcBlockBytes = 8 * kQcCols * 2;      // 8 rows of 128 bytes
constexpr uint32_t kQcSegs = kQcRows / 16;               // 16-row segments per column

__device__ __forceinline__ uint32_t qc_offset(uint32_t row, uint32_t chunk)
{
    const uint32_t b = row >> 3;
    return b * kQcBlockBytes + (row & 7) * (kQcCols * 2) + ((chunk ^ (b >> 1)) & 7) * 16;
}

// hardware converters with a compile-time byte selector
template <int SEL>
__device__ __forceinline__ uint32_t hw_enc_bf16(uint32_t old, uint32_t pair, float scale)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(old, __builtin_bit_cast(bf16x2, pair), scale, SEL);
}
template <int SEL>
__device__ __forceinline__ uint32_t hw_enc_f32(uint32_t old, float a0, float a1)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a0, a1, 1.0f, SEL);
}
// ---- stochastic rounding on the converter -----------------------------------
// The rule: with g_k <= |a| < g_{k+1} (neighbouring E2M1 magnitudes) and
// T = floor((|a| - g_k) / (g_{k+1} - g_k) * 2^16), the element rounds up
// exactly when its 16-bit draw r16 < T; |a| >= 6 encodes 6; the sign is kept.
//
// v_cvt_scalef32_sr_pk_fp4_f32 (scale 1) encodes its first value with the
// random word R as: up exactly when floor(f * 2^32) + R >= 2^32, f the same
// fraction (|a| >= 6 gives 6, sign kept).  This was measured on the device for
// 2^17 random value / word pairs, all in agreement.  With R = (0xFFFF - r16)
// << 16 the carry happens exactly when (T + 0xFFFF - r16) * 2^16 plus the low
// 16 bits of floor(f * 2^32) reaches 2^32, i.e. when T + 0xFFFF - r16 >= 2^16,
// i.e. when r16 < T: the rule.  The second value of the pair is +0, which
// encodes to 0 whatever R is, so each conversion serves one element.
//
// The converter writes byte 0 of its destination only (nibbles: first value,
// second value) and keeps the other three bytes, which the compiler does not
// model as an input: they hold whatever the register held, and only byte 0
// of the result is ever used.
__device__ __forceinline__ uint32_t hw_sr_byte(float a, uint32_t R)
{
    return __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, (f32x2){a, 0.0f}, R, 1.0f, 0);
}

template <int SEL>
__device__ __forceinline__ uint32_t hw_dec_bf16(uint32_t codes, float scale)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, SEL));
}
template <int SEL>
__device__ __forceinline__ uint32_t hw_dec_nv(uint32_t codes, float s_eff)
{
    const f32x2 g = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, SEL);
    return bf16_pair_rne(g[0] * s_eff, g[1] * s_eff);
}

// Dequantize 8 codes (one 32-bit word, element i in nibble i) to 4 BF16 pairs.
template <int FMT>
__device__ __forceinline__ void decode8(uint32_t cw, float s_eff, uint32_t *yp)
{
    if (FMT == FMT_MX) {
        yp[0] = hw_dec_bf16<0>(cw, s_eff);
        yp[1] = hw_dec_bf16<1>(cw, s_eff);
        yp[2] = hw_dec_bf16<2>(cw, s_eff);
        yp[3] = hw_dec_bf16<3>(cw, s_eff);
    } else {
        yp[0] = hw_dec_nv<0>(cw, s_eff);
        yp[1] = hw_dec_nv<1>(cw, s_eff);
        yp[2] = hw_dec_nv<2>(cw, s_eff);
        yp[3] = hw_dec_nv<3>(cw, s_eff);
    }
}

// ---- the block-part encoder ------------------------------------------------
// xp: NP packed BF16 pairs along the quantization axis (element 2i in the low
// half of xp[i]), NP = 4 (8 elements) or 8 (16 elements); rnd: Philox output
// blocks for elements 0-7 and 8-15 (SR only).
// Outputs: cw (element 2i in the low nibble of byte i, 8 codes per word) and
// yp (the dequantized BF16 values, packed like xp).
template <int FMT, int RND, int NP>
__device__ __forceinline__ void encode_pairs(const uint32_t (&xp)[NP], const BlockScale &b,
                                             const u32x4 *rnd, uint32_t (&cw)[NP / 4],
                                             uint32_t (&yp)[NP])
{
    constexpr int NW = NP / 4;
    if (FMT == FMT_MX && RND == RND_RNE) {
        // hardware encode straight from BF16 at the power-of-two scale
#pragma unroll
        for (int h = 0; h < NW; ++h) {
            uint32_t c = hw_enc_bf16<0>(0u, xp[4 * h + 0], b.s_eff);
            c = hw_enc_bf16<1>(c, xp[4 * h + 1], b.s_eff);
            c = hw_enc_bf16<2>(c, xp[4 * h + 2], b.s_eff);
            c = hw_enc_bf16<3>(c, xp[4 * h + 3], b.s_eff);
            cw[h] = c;
        }
    } else {
        float a[2 * NP];
        if (FMT == FMT_MX) {
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                a[2 * i] = __builtin_fabsf(as_f(lo_bits(xp[i]))) * b.rcp;
                a[2 * i + 1] = __builtin_fabsf(as_f(hi_bits(xp[i]))) * b.rcp;
            }
        } else if (b.xs == 1.0f) {
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                a[2 * i] = div_corrected(__builtin_fabsf(as_f(lo_bits(xp[i]))), b.sq, b.rcp);
                a[2 * i + 1] = div_corrected(__builtin_fabsf(as_f(hi_bits(xp[i]))), b.sq, b.rcp);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                a[2 * i] = div_corrected(__builtin_fabsf(as_f(lo_bits(xp[i]))) * b.xs, b.sq, b.rcp);
                a[2 * i + 1] = div_corrected(__builtin_fabsf(as_f(hi_bits(xp[i]))) * b.xs, b.sq, b.rcp);
            }
        }
        // signed quotients
        float sa[2 * NP];
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            sa[2 * i] = as_f(as_u(a[2 * i]) | ((xp[i] << 16) & 0x80000000u));
            sa[2 * i + 1] = as_f(as_u(a[2 * i + 1]) | (xp[i] & 0x80000000u));
        }
        if (RND == RND_RNE) {
            // hardware RNE encoder at scale 1
#pragma unroll
            for (int h = 0; h < NW; ++h) {
                uint32_t c = hw_enc_f32<0>(0u, sa[8 * h + 0], sa[8 * h + 1]);
                c = hw_enc_f32<1>(c, sa[8 * h + 2], sa[8 * h + 3]);
                c = hw_enc_f32<2>(c, sa[8 * h + 4], sa[8 * h + 5]);
                c = hw_enc_f32<3>(c, sa[8 * h + 6], sa[8 * h + 7]);
                cw[h] = c;
            }
        } else {
            // hardware SR encoder, one element per conversion; pair i draws
            // from word i & 3 of Philox block i >> 2, element 2i from its low
            // half and 2i + 1 from its high half.  Byte 0 of pb[k] is the code
            // byte of pair 4h + k (upper bytes undefined); v_perm gathers them.
#pragma unroll
            for (int h = 0; h < NW; ++h) {
                uint32_t pb[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int i = 4 * h + k;
                    const uint32_t nw = ~rnd[h].v[k];          // 0xFFFF - r16 in each half
                    const uint32_t e = hw_sr_byte(sa[2 * i], nw << 16);
                    const uint32_t o = hw_sr_byte(sa[2 * i + 1], nw & 0xFFFF0000u);
                    pb[k] = (o << 4) | e;
                }
                cw[h] = __builtin_amdgcn_perm(pb[1], pb[0], 0x0C0C0400u) |
                        __builtin_amdgcn_perm(pb[3], pb[2], 0x04000C0Cu);
            }
        }
    }
#pragma unroll
    for (int h = 0; h < NW; ++h) decode8<FMT>(cw[h], b.s_eff, &yp[4 * h]);
}

// Clip mask of 2*NP elements (bit j set when element j has a <= 6, i.e. kept).
template <int FMT, int NP>
__device__ __forceinline__ uint32_t keep_mask(const uint32_t (&xp)[NP], const BlockScale &b)
{
    uint32_t k = 0;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        k |= (scaled_mag<FMT>(lo_bits(xp[i]), b) <= 6.0f ? 1u : 0u) << (2 * i);
        k |= (scaled_mag<FMT>(hi_bits(xp[i]), b) <= 6.0f ? 1u : 0u) << (2 * i + 1);
    }
    return k;
}


// ---- workgroup maximum and the per-tensor NVFP4 scale ----------------------
template <int NT>
__device__ __forceinline__ uint32_t block_reduce_max(uint32_t m, uint32_t *red)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        m = max(m, (uint32_t)__shfl_xor((int)m, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) m = max(m, red[w]);
    return m;
}

// NVFP4 per-tensor outer scale from the partial maxima (every thread of a
// workgroup of NT threads; NT must be the launching workgroup's size, which
// sizes the per-wave slots of the reduction).
template <int NT>
__device__ __forceinline__ OuterScale tensor_scale(const uint32_t *__restrict__ partials,
                                                   uint32_t npart)
{
    static_assert(NT % 64 == 0 && NT <= 1024, "whole waves, at most 16");
    __shared__ uint32_t red[NT / 64];
    uint32_t m = 0;
    for (uint32_t i = threadIdx.x; i < npart; i += NT) m = max(m, partials[i]);
    m = block_reduce_max<NT>(m, red);
    return make_outer(as_f(m << 16));
}

// Halves of a packed BF16 pair word (elements 2w, 2w + 1 of a chunk) whose
// bit is set in the 8-bit mask r (bit e for element e of the chunk).
__device__ __forceinline__ uint32_t retained_halves(uint32_t r, int e0)
{
    return (((r >> e0) & 1u) ? 0xFFFFu : 0u) | (((r >> (e0 + 1)) & 1u) ? 0xFFFF0000u : 0u);
}

// FP8 E4M3 fake quantization of a packed BF16 pair under two channel scales
// (each a BlockScale: s_eff and the correctly rounded quotient's reciprocal):
// a = RN(|x| / s), E4M3 nearest-even saturating at 448, value * s, sign kept;
// a zero scale gives +-0.  clip0 / clip1 are set when a > 448.  The E4M3
// rounding is gfx950's FP8 converter applied to min(a, 448), decoded exactly
// by the FP8 -> FP32 converter: this equals the nearest-even, saturating
// encoder for every non-negative FP32 value (checked on the device for every
// value below 2^11 and a sample above, +inf and NaN included).
__device__ __forceinline__ uint32_t fp8_fake_pair(uint32_t xpair, const BlockScale &s0,
                                                  const BlockScale &s1, bool *clip0, bool *clip1)
{
    const uint32_t x0 = lo_bits(xpair), x1 = hi_bits(xpair);
    const float a0 = div_corrected(as_f(x0 & 0x7FFFFFFFu) * s0.xs, s0.sq, s0.rcp);
    const float a1 = div_corrected(as_f(x1 & 0x7FFFFFFFu) * s1.xs, s1.sq, s1.rcp);
    *clip0 = a0 > 448.0f;
    *clip1 = a1 > 448.0f;
    const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fminf(a0, 448.0f),
                                                   __builtin_fminf(a1, 448.0f), 0, false);
    const float m0 = __builtin_amdgcn_cvt_f32_fp8(pk, 0) * s0.s_eff;
    const float m1 = __builtin_amdgcn_cvt_f32_fp8(pk, 1) * s1.s_eff;
    return bf16_pair_rne(as_f(as_u(m0) | (x0 & 0x80000000u)), as_f(as_u(m1) | (x1 & 0x80000000u)));
}

}  // namespace fqdev
