/*
 * fq_oracle.c -- reference implementation of blockwise FP4 fake quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the GPU library is
 * checked against.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load it.  The product path never calls it and shares
 * no code, header, table or helper with it.
 *
 * It is written to be read, not to be fast: scalar loops, one element at a
 * time, every rounding step spelled out.  Each function names the passage it
 * follows.  Sources (cited by title and section):
 *
 *  [TJ2]   "Resumo Tecnico: TetraJet-v2" (gist.science, paper 2510.27527),
 *          sec. 2.A "Quantizacao Dupla de Blocos Nao Viciada para Camadas
 *          Lineares NVFP4": NVFP4 groups of 16 elements with an 8-bit scale, a
 *          128-element outer block with its own scale over 16-element inner
 *          blocks, stochastic rounding with E[round(x)] = x in the backward
 *          pass, 1x16 weight groups aligned for the transposed weight.
 *          sec. 1 "Declaracao do Problema": adjacent FP4 bins 0 and 0.5.
 *  [GPTOSS] "Aprimorando gpt-oss para Precisao e Desempenho com Treinamento
 *          Consciente a Quantizacao" (brainai.pro), "O que ha de novo": MXFP4
 *          vs NVFP4, NVFP4 carries an FP8 E4M3 scale.
 *  [GPTOSS-EN] gpt-oss fine-tuning with QAT tutorial (thakicloud), section
 *          "NVFP4: The Next Generation" / "NVFP4 Advantages": E4M3 scaling.
 *  [QATREC] "Como o Treinamento com Quantizacao Detecta e Recupera Precisao em
 *          Inferencia de Baixa Precisao" (brainai.pro), "Detalhes tecnicos ou
 *          Implementacao": fake quantization (quantize/dequantize inside a
 *          wider type) in the forward pass, gradients through the quantizer by
 *          the straight-through estimator, exposing rounding and clipping.
 *  [MX]    OCP Microscaling Formats (MX) Specification v1.0: FP4 E2M1 element
 *          encoding (sec. 5.3.3), E8M0 scale (sec. 5.4.1), shared scale
 *          2^(floor(log2(amax)) - emax_elem) with emax_elem = 2 for E2M1
 *          (sec. 6.3).
 *  [OFP8]  OCP 8-bit Floating Point Specification (OFP8) v1.0: E4M3 encoding,
 *          bias 7, no infinities, largest finite 448.
 *  [PHILOX] J. Salmon, M. Moraes, R. Dror, D. Shaw, "Parallel Random Numbers:
 *          As Easy as 1, 2, 3", SC'11, sec. 3.2 (Philox), Philox4x32-10.
 *
 * Readings where the sources leave a step open are marked READING below.
 * Precision: the formats fix their scales as FP32 (outer scales) and E4M3 /
 * E8M0 (block scales); the quotient x / s that decides each FP4 code is taken
 * in FP32 as well, so every decision is made in IEEE binary32 with
 * round-to-nearest-even.  Build with -ffp-contract=off and no -ffast-math so
 * that every float expression below is a single correctly rounded operation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* Format identifiers used by this file (its own, not the library's). */
/* ------------------------------------------------------------------ */
enum { FQO_MX = 0, FQO_NV_TENSOR = 1, FQO_NV_BLOCK128 = 2 };
enum { FQO_RNE = 0, FQO_SR = 1 };

/* ------------------------------------------------------------------ */
/* BF16 <-> FP32                                                      */
/* ------------------------------------------------------------------ */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* BF16 is the upper half of an FP32 word: widening is exact. */
float fqo_bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* FP32 -> BF16, round to nearest, ties to even, written as "pick the nearer of
 * the two neighbouring BF16 values".  lo is f with the low 16 bits cleared
 * (toward zero); hi is the next BF16 value away from zero.  Past the largest
 * finite BF16 the next value is infinity, which for rounding purposes sits at
 * 2^128 (IEEE 754 overflow rule).  The distances are exact in double.
 * Non-finite input is out of contract (NaN stays NaN, infinities stay). */
uint16_t fqo_f32_to_bf16(float f)
{
    uint32_t u = bits_from_f32(f);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u);
    if (isinf(f)) return (uint16_t)(u >> 16);
    uint16_t lo_bits = (uint16_t)(u >> 16);
    uint16_t hi_bits = (uint16_t)(lo_bits + 1);      /* next magnitude up */
    double lo = fqo_bf16_to_f32(lo_bits);
    double hi = fqo_bf16_to_f32(hi_bits);
    if (isinf(hi)) hi = copysign(ldexp(1.0, 128), hi);
    double x = f;
    double dlo = fabs(x - lo);
    double dhi = fabs(hi - x);
    if (dlo < dhi) return lo_bits;
    if (dhi < dlo) return hi_bits;
    return (lo_bits & 1u) ? hi_bits : lo_bits;       /* tie: even mantissa */
}

/* ------------------------------------------------------------------ */
/* FP4 E2M1 element  ([MX] sec. 5.3.3; grid also implied by [TJ2] sec. 1) */
/* ------------------------------------------------------------------ */

/* Magnitudes of the eight non-negative E2M1 codes: sign bit 3, two exponent
 * bits with bias 1, one mantissa bit; exponent 0 is subnormal (0 and 0.5). */
static const double E2M1_GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double fqo_e2m1_decode(int code)
{
    double m = E2M1_GRID[code & 7];
    return (code & 8) ? -m : m;
}

/* Round a non-negative magnitude to the nearest E2M1 grid value; on a tie take
 * the code whose mantissa bit (bit 0) is 0 ("round to nearest even").  Values
 * beyond 6 land on 6, the largest code, since E2M1 has no infinity.  The
 * search is brute force over the eight magnitudes. */
int fqo_e2m1_rne(float a)
{
    if ((double)a >= 6.0) return 7;     /* at or past the top of the grid */
    int best = 0;
    double bestd = fabs((double)a - E2M1_GRID[0]);
    for (int m = 1; m < 8; ++m) {
        double d = fabs((double)a - E2M1_GRID[m]);
        if (d < bestd || (d == bestd && (m & 1) == 0 && (best & 1) == 1)) {
            best = m;
            bestd = d;
        }
    }
    return best;
}

/* Stochastic rounding of a non-negative magnitude with one 16-bit draw r.
 * [TJ2] sec. 2.A asks only for E[round(x)] = x.  READING: take the bracketing
 * grid values g_k <= a < g_{k+1}, the exact fraction f = (a - g_k) /
 * (g_{k+1} - g_k), the integer threshold T = floor(f * 65536), and round up
 * when r < T, so P(up) = T / 65536 (equal to f whenever f * 2^16 is an
 * integer, short of it by less than 2^-16 otherwise).  a >= 6 is clipped to 6. */
int fqo_e2m1_sr(float a, uint16_t r)
{
    if ((double)a >= 6.0) return 7;
    int k = 0;
    while (k < 6 && E2M1_GRID[k + 1] <= (double)a) ++k;
    double f = ((double)a - E2M1_GRID[k]) / (E2M1_GRID[k + 1] - E2M1_GRID[k]);
    uint32_t T = (uint32_t)floor(f * 65536.0);
    return k + (((uint32_t)r < T) ? 1 : 0);
}

/* ------------------------------------------------------------------ */
/* E8M0 scale ([MX] sec. 5.4.1, 6.3)                                  */
/* ------------------------------------------------------------------ */

float fqo_e8m0_decode(uint8_t code)
{
    if (code == 255) return NAN;
    return (float)ldexp(1.0, (int)code - 127);
}

/* Shared MX scale exponent for a block maximum: floor(log2(amax)) - 2, where
 * 2 is the exponent of the largest E2M1 value (6 = 1.5 * 2^2).  READING: the
 * code is clamped to 0..254 (2^-127 .. 2^127); a zero block takes code 0 and
 * 255 (NaN) is never produced.  floor(log2) is read exactly from frexp. */
uint8_t fqo_mx_scale_code(float amax)
{
    int k;
    if (amax == 0.0f) {
        k = -127;
    } else {
        int e;
        frexp((double)amax, &e);          /* amax = f * 2^e, 0.5 <= f < 1 */
        k = (e - 1) - 2;
        if (k < -127) k = -127;
        if (k > 127) k = 127;
    }
    return (uint8_t)(k + 127);
}

/* ------------------------------------------------------------------ */
/* E4M3 scale ([OFP8]; NVFP4 block scale per [GPTOSS], [TJ2] sec. 2.A) */
/* ------------------------------------------------------------------ */

double fqo_e4m3_decode(uint8_t code)
{
    int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);            /* subnormal: m * 2^-9 */
    else v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* Non-negative value -> E4M3, nearest, ties to the even code, saturating at
 * 448 (code 0x7E).  READING: scales are rounded to nearest (not up); values at
 * or beyond 448 saturate.  Brute force over the 127 finite non-negative codes. */
uint8_t fqo_e4m3_encode(float v)
{
    if (!(v > 0.0f)) return 0;
    if ((double)v >= 448.0) return 0x7E;
    int best = 0;
    double bestd = fabs((double)v);
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs((double)v - fqo_e4m3_decode((uint8_t)c));
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return (uint8_t)best;
}

/* ------------------------------------------------------------------ */
/* Philox4x32-10 ([PHILOX] sec. 3.2)                                  */
/* ------------------------------------------------------------------ */

void fqo_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2],
                       uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u; /* round multipliers */
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u; /* key (Weyl) increments */
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { k0 += W0; k1 += W1; }
        uint64_t p0 = (uint64_t)M0 * c0;
        uint64_t p1 = (uint64_t)M1 * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The 16-bit draw for element n (row-major index in the orientation being
 * quantized).  READING: key = (seed low word, seed high word); counter =
 * (low and high words of n / 8, 0, 0); one call feeds eight consecutive
 * elements, element n taking 16-bit half (n mod 2) of output word
 * (n / 2) mod 4, low half first. */
uint16_t fqo_r16(uint64_t seed, uint64_t n)
{
    uint64_t call = n >> 3;
    uint32_t ctr[4] = {(uint32_t)call, (uint32_t)(call >> 32), 0u, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t o[4];
    fqo_philox4x32_10(ctr, key, o);
    uint32_t w = o[(n >> 1) & 3];
    return (uint16_t)((n & 1) ? (w >> 16) : (w & 0xFFFFu));
}

/* ------------------------------------------------------------------ */
/* Block scales                                                       */
/* ------------------------------------------------------------------ */

/* NVFP4 second-level scale from a magnitude that the first level must cover:
 * the largest E2M1 value (6) times the largest E4M3 value (448) = 2688.
 * Used for the per-tensor scale (amax of the tensor) and, READING, in the same
 * form for the per-128-element outer scale of [TJ2] sec. 2.A. */
float fqo_nv_outer_scale(float amax) { return amax / 2688.0f; }

/* NVFP4 block scale: the block needs amax_b / 6 expressed in units of the
 * outer scale s, stored as E4M3; the effective scale is that E4M3 value times
 * s, in FP32.  READING: each of the two divisions and the product is one FP32
 * operation rounded to nearest; s = 0 (all-zero tensor or outer block) gives
 * a zero block scale. */
static void nv_block_scale(float amax_b, float s, uint8_t *e4_out, float *s_eff_out)
{
    float sc = 0.0f;
    if (s != 0.0f) {
        float per_block = amax_b / 6.0f;
        sc = per_block / s;
    }
    uint8_t e4 = fqo_e4m3_encode(sc);
    *e4_out = e4;
    *s_eff_out = (float)fqo_e4m3_decode(e4) * s;
}

/* Scaled magnitude a = |x| / s_eff in FP32; a zero scale maps to a = 0. */
static float scaled_magnitude(float x, float s_eff)
{
    if (s_eff == 0.0f) return 0.0f;
    return fabsf(x) / s_eff;
}

/* Dequantized element: BF16(RN(+-g * s_eff)); the sign of the code is kept,
 * so a negative input that rounds to zero dequantizes to -0.0 (READING). */
static uint16_t dequant_element(int code, float s_eff)
{
    float mag = (float)E2M1_GRID[code & 7] * s_eff;
    float v = (code & 8) ? -mag : mag;
    return fqo_f32_to_bf16(v);
}

static int block_size_of(int fmt) { return fmt == FQO_MX ? 32 : 16; }

/* ------------------------------------------------------------------ */
/* Fake quantization along rows                                        */
/* ------------------------------------------------------------------ */

/* Per-tensor absolute maximum of a BF16 tensor (exact). */
float fqo_absmax(const uint16_t *x, int64_t n)
{
    float A = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float v = fabsf(fqo_bf16_to_f32(x[i]));
        if (v > A) A = v;
    }
    return A;
}

/*
 * Quantize an R x C BF16 tensor in 1xB groups along each row (the contiguous
 * axis), B = 32 for MXFP4 and 16 for NVFP4, and dequantize it back.
 *
 * Outputs (any may be NULL):
 *   codes  [R, C/2]   two E2M1 codes per byte, element 2j in the low nibble
 *   scales [R, C/B]   E8M0 (MX) or E4M3 (NV) block scale codes
 *   outer             NV per-tensor: 1 float; NV 128-block: [R, C/128] floats
 *   y      [R, C]     dequantized BF16
 *   clip   [R, C]     1 where the scaled magnitude exceeds 6 (the element was
 *                     clipped), else 0
 * Stochastic rounding draws fqo_r16(seed, index_base + r * C + c) for element
 * (r, c): index_base = 0 for a whole tensor, or the flat index of the first
 * element when x is a run of whole rows cut from a larger tensor (a sample;
 * the per-tensor format then takes its maximum over the sample only).
 * Returns 0, or -1 for a shape the format cannot block.
 */
int fqo_quantize_rows_at(int fmt, int rounding, uint64_t seed, uint64_t index_base,
                         const uint16_t *x, int64_t R, int64_t C,
                         uint8_t *codes, uint8_t *scales, float *outer,
                         uint16_t *y, uint8_t *clip, int nthreads)
{
    const int B = block_size_of(fmt);
    if (R <= 0 || C <= 0 || C % B != 0) return -1;
    if (fmt == FQO_NV_BLOCK128 && C % 128 != 0) return -1;

    float s_tensor = 0.0f;
    if (fmt == FQO_NV_TENSOR) {
        s_tensor = fqo_nv_outer_scale(fqo_absmax(x, R * C));
        if (outer) outer[0] = s_tensor;
    }
    (void)nthreads;

#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
#endif
    for (int64_t r = 0; r < R; ++r) {
        const uint16_t *xr = x + r * C;
        float s_outer = s_tensor;
        for (int64_t b0 = 0; b0 < C; b0 += B) {
            /* outer scale of the 128-element block holding this inner block */
            if (fmt == FQO_NV_BLOCK128 && b0 % 128 == 0) {
                float amax128 = 0.0f;
                for (int64_t c = b0; c < b0 + 128; ++c) {
                    float v = fabsf(fqo_bf16_to_f32(xr[c]));
                    if (v > amax128) amax128 = v;
                }
                s_outer = fqo_nv_outer_scale(amax128);
                if (outer) outer[r * (C / 128) + b0 / 128] = s_outer;
            }

            float amax_b = 0.0f;
            for (int64_t c = b0; c < b0 + B; ++c) {
                float v = fabsf(fqo_bf16_to_f32(xr[c]));
                if (v > amax_b) amax_b = v;
            }

            uint8_t scode;
            float s_eff;
            if (fmt == FQO_MX) {
                scode = fqo_mx_scale_code(amax_b);
                s_eff = fqo_e8m0_decode(scode);
            } else {
                nv_block_scale(amax_b, s_outer, &scode, &s_eff);
            }
            if (scales) scales[r * (C / B) + b0 / B] = scode;

            for (int64_t c = b0; c < b0 + B; ++c) {
                float xv = fqo_bf16_to_f32(xr[c]);
                float a = scaled_magnitude(xv, s_eff);
                int m;
                if (rounding == FQO_SR)
                    m = fqo_e2m1_sr(a, fqo_r16(seed, index_base + (uint64_t)(r * C + c)));
                else
                    m = fqo_e2m1_rne(a);
                int code = (signbit(xv) ? 8 : 0) | m;
                if (codes) {
                    uint8_t *p = &codes[r * (C / 2) + c / 2];
                    if ((c & 1) == 0) *p = (uint8_t)((*p & 0xF0) | code);
                    else *p = (uint8_t)((*p & 0x0F) | (code << 4));
                }
                if (y) y[r * C + c] = dequant_element(code, s_eff);
                if (clip) clip[r * C + c] = (uint8_t)(a > 6.0f);
            }
        }
    }
    return 0;
}

int fqo_quantize_rows(int fmt, int rounding, uint64_t seed,
                      const uint16_t *x, int64_t R, int64_t C,
                      uint8_t *codes, uint8_t *scales, float *outer,
                      uint16_t *y, uint8_t *clip, int nthreads)
{
    return fqo_quantize_rows_at(fmt, rounding, seed, 0, x, R, C, codes, scales, outer, y, clip,
                                nthreads);
}

/* ------------------------------------------------------------------ */
/* Static outlier-channel retention ([TJ2] sec. 2.C, "Retencao Estatica */
/* de Outliers"): a fixed set of channels stays in FP8 in the forward   */
/* pass while the rest is FP4.                                          */
/* ------------------------------------------------------------------ */

/* FP8 E4M3 fake quantization of one element under its channel's FP32 scale.
 * READING: a = |x| / s in FP32, E4M3 round-to-nearest-even saturating at 448
 * ([OFP8]; the same encoder as the NVFP4 block scale), value = dec(e) * s in
 * FP32, sign of x kept, then BF16; a zero channel scale gives +-0. */
static uint16_t fp8_fake_quant(float xv, float s)
{
    float mag = 0.0f;
    if (s != 0.0f) {
        float a = fabsf(xv) / s;
        mag = (float)fqo_e4m3_decode(fqo_e4m3_encode(a)) * s;
    }
    return fqo_f32_to_bf16(signbit(xv) ? -mag : mag);
}

/* Element-wise FP8 fake quantization of n BF16 values, each under its own
 * scale s[i] (the retained channel's), and the straight-through clip flag of
 * each.  READING: an FP8 element is clipped when a = |x| / s (FP32) exceeds
 * 448, the largest E4M3 value, as an FP4 element is when a exceeds 6. */
int fqo_fp8_fake(const uint16_t *x, const float *s, int64_t n, uint16_t *y, uint8_t *clip)
{
    for (int64_t i = 0; i < n; ++i) {
        float xv = fqo_bf16_to_f32(x[i]);
        y[i] = fp8_fake_quant(xv, s[i]);
        if (clip) clip[i] = (s[i] != 0.0f && fabsf(xv) / s[i] > 448.0f) ? 1 : 0;
    }
    return 0;
}

/* Row-axis fake quantization with retained channels.  retain[c] != 0 marks
 * column c as an FP8 channel with scale chan_scale[c].  READING: retained
 * elements take no part in the FP4 scales (block and 128-element outer
 * maxima are taken over the other elements), carry FP4 code 0, and their y is
 * the FP8 fake quantization above.  Only the MXFP4 and double-block NVFP4
 * formats (no tensor-wide FP4 scale to redefine).  The stochastic-rounding
 * index of an FP4 element is r * C + c as in fqo_quantize_rows. */
int fqo_quantize_rows_retain(int fmt, int rounding, uint64_t seed,
                             const uint16_t *x, int64_t R, int64_t C,
                             const uint8_t *retain, const float *chan_scale,
                             uint8_t *codes, uint8_t *scales, float *outer,
                             uint16_t *y, int nthreads)
{
    const int B = block_size_of(fmt);
    if (fmt == FQO_NV_TENSOR) return -1;
    if (R <= 0 || C <= 0 || C % B != 0) return -1;
    if (fmt == FQO_NV_BLOCK128 && C % 128 != 0) return -1;
    (void)nthreads;

#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
#endif
    for (int64_t r = 0; r < R; ++r) {
        const uint16_t *xr = x + r * C;
        float s_outer = 0.0f;
        for (int64_t b0 = 0; b0 < C; b0 += B) {
            if (fmt == FQO_NV_BLOCK128 && b0 % 128 == 0) {
                float amax128 = 0.0f;
                for (int64_t c = b0; c < b0 + 128; ++c) {
                    if (retain[c]) continue;
                    float v = fabsf(fqo_bf16_to_f32(xr[c]));
                    if (v > amax128) amax128 = v;
                }
                s_outer = fqo_nv_outer_scale(amax128);
                if (outer) outer[r * (C / 128) + b0 / 128] = s_outer;
            }
            float amax_b = 0.0f;
            for (int64_t c = b0; c < b0 + B; ++c) {
                if (retain[c]) continue;
                float v = fabsf(fqo_bf16_to_f32(xr[c]));
                if (v > amax_b) amax_b = v;
            }
            uint8_t scode;
            float s_eff;
            if (fmt == FQO_MX) {
                scode = fqo_mx_scale_code(amax_b);
                s_eff = fqo_e8m0_decode(scode);
            } else {
                nv_block_scale(amax_b, s_outer, &scode, &s_eff);
            }
            if (scales) scales[r * (C / B) + b0 / B] = scode;
            for (int64_t c = b0; c < b0 + B; ++c) {
                float xv = fqo_bf16_to_f32(xr[c]);
                int code = 0;
                uint16_t yv;
                if (retain[c]) {
                    yv = fp8_fake_quant(xv, chan_scale[c]);
                } else {
                    float a = scaled_magnitude(xv, s_eff);
                    int m = (rounding == FQO_SR)
                                ? fqo_e2m1_sr(a, fqo_r16(seed, (uint64_t)(r * C + c)))
                                : fqo_e2m1_rne(a);
                    code = (signbit(xv) ? 8 : 0) | m;
                    yv = dequant_element(code, s_eff);
                }
                if (codes) {
                    uint8_t *p = &codes[r * (C / 2) + c / 2];
                    if ((c & 1) == 0) *p = (uint8_t)((*p & 0xF0) | code);
                    else *p = (uint8_t)((*p & 0x0F) | (code << 4));
                }
                if (y) y[r * C + c] = yv;
            }
        }
    }
    return 0;
}

/* Effective scale of one block from stored scale codes (and outer scales). */
static float stored_block_scale(int fmt, const uint8_t *scales, const float *outer,
                                int64_t r, int64_t c, int64_t C)
{
    const int B = block_size_of(fmt);
    uint8_t scode = scales[r * (C / B) + c / B];
    if (fmt == FQO_MX) return fqo_e8m0_decode(scode);
    float s = (fmt == FQO_NV_TENSOR) ? outer[0] : outer[r * (C / 128) + c / 128];
    return (float)fqo_e4m3_decode(scode) * s;
}

/* Dequantize codes + scales (+ outer scales), row layout as produced above. */
int fqo_dequantize_rows(int fmt, const uint8_t *codes, const uint8_t *scales,
                        const float *outer, int64_t R, int64_t C, uint16_t *y,
                        int nthreads)
{
    const int B = block_size_of(fmt);
    if (R <= 0 || C <= 0 || C % B != 0) return -1;
    if (fmt == FQO_NV_BLOCK128 && C % 128 != 0) return -1;
    (void)nthreads;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
#endif
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t c = 0; c < C; ++c) {
            float s_eff = stored_block_scale(fmt, scales, outer, r, c, C);
            uint8_t byte = codes[r * (C / 2) + c / 2];
            int code = (c & 1) ? (byte >> 4) : (byte & 0x0F);
            y[r * C + c] = dequant_element(code, s_eff);
        }
    }
    return 0;
}

/* Straight-through estimator with clipping ([QATREC], "Detalhes tecnicos"):
 * the gradient passes unchanged through the quantizer except where the
 * forward clipped the element.  READING: "clipped" means the FP32 scaled
 * magnitude |x| / s_eff, recomputed from x and the forward's stored scales,
 * exceeds 6; there the gradient is +0. */
int fqo_ste_backward_rows(int fmt, const uint16_t *x, const uint8_t *scales,
                          const float *outer, const uint16_t *dy, int64_t R,
                          int64_t C, uint16_t *dx, int nthreads)
{
    const int B = block_size_of(fmt);
    if (R <= 0 || C <= 0 || C % B != 0) return -1;
    if (fmt == FQO_NV_BLOCK128 && C % 128 != 0) return -1;
    (void)nthreads;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
#endif
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t c = 0; c < C; ++c) {
            float s_eff = stored_block_scale(fmt, scales, outer, r, c, C);
            float a = scaled_magnitude(fqo_bf16_to_f32(x[r * C + c]), s_eff);
            dx[r * C + c] = (a > 6.0f) ? (uint16_t)0 : dy[r * C + c];
        }
    }
    return 0;
}

/* Random Hadamard transform along rows, in blocks of n = 16 or 128
 * consecutive elements ("Resumo Tecnico: TetraJet-v2", sec. 2.C OutControl:
 * a random Hadamard transform is applied to the backward's products so that
 * outlier energy spreads over the channels before quantization).
 *
 * Random signs: position j along the row (the column index) has sign -1
 * when bit (j mod 128) of Philox4x32-10(key = seed, counter = (j / 128, 0,
 * 0, 0)) is set (bit t of output word w counts as bit 32w + t), else +1.
 * Transform of a block v = s o x (exact sign flips of the BF16 values,
 * widened to FP32): radix-2 butterflies in FP32 with half-widths h = 1, 2,
 * 4, ..., n/2, each pair (i, i + h) of a 2h-group becoming (a + b, a - b);
 * this is the Hadamard matrix in Sylvester order.  Then y = BF16_RNE(
 * RN32(c_n * v)) with c_n the FP32 value nearest to 1/sqrt(n) (0.25 for n =
 * 16).  The rows of a [R, C] tensor are independent. */
int fqo_rht_sign_bit(uint64_t seed, uint64_t j)
{
    const uint32_t ctr[4] = {(uint32_t)(j >> 7), (uint32_t)(j >> 39), 0u, 0u};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t o[4];
    fqo_philox4x32_10(ctr, key, o);
    const unsigned b = (unsigned)(j & 127);
    return (int)((o[b >> 5] >> (b & 31)) & 1u);
}

int fqo_hadamard_rows(const uint16_t *x, int64_t R, int64_t C, int n, uint64_t seed,
                      float c_n, uint16_t *y, int nthreads)
{
    if (R <= 0 || C <= 0 || (n != 16 && n != 128) || C % n != 0) return -1;
    uint8_t *neg = (uint8_t *)malloc((size_t)C);     /* the sign of each column */
    if (!neg) return -2;
    for (int64_t j = 0; j < C; ++j) neg[j] = (uint8_t)fqo_rht_sign_bit(seed, (uint64_t)j);
    (void)nthreads;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
#endif
    for (int64_t r = 0; r < R; ++r) {
        float v[128];
        for (int64_t b0 = 0; b0 < C; b0 += n) {
            for (int i = 0; i < n; ++i) {
                float e = fqo_bf16_to_f32(x[r * C + b0 + i]);
                v[i] = neg[b0 + i] ? -e : e;
            }
            for (int h = 1; h < n; h *= 2)
                for (int g = 0; g < n; g += 2 * h)
                    for (int t = g; t < g + h; ++t) {
                        float a = v[t], b = v[t + h];
                        v[t] = a + b;
                        v[t + h] = a - b;
                    }
            for (int i = 0; i < n; ++i) y[r * C + b0 + i] = fqo_f32_to_bf16(c_n * v[i]);
        }
    }
    free(neg);
    return 0;
}

int fqo_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
