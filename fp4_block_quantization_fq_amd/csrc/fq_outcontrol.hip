// fq_outcontrol.hip -- TetraJet-v2's two training-time controls on gfx950.
//
// "Resumo Tecnico: TetraJet-v2", sec. 2.B (OsciReset): a weight oscillates
// when its quantized value keeps travelling between bins while the master
// weight barely moves; the risk is the ratio of the two distances travelled,
// and at a low learning rate an oscillating master weight is reset to the
// centre of its current quantization bin.  Sec. 2.C (OutControl, static
// outlier retention): the few channels with large norms, found once during a
// calibration window, stay in FP8 in the forward and backward passes while
// the rest is FP4.
//
// All of it is elementwise or per-channel streaming work:
//  * k_osci_track / k_osci_reset: four weights per lane (16-byte FP32 and
//    8-byte BF16 accesses), FP32 distances, one rounding per operation.
//  * k_channel_absmax: the calibration statistic, the maximum magnitude of
//    each column, folded into a running per-channel maximum with integer
//    atomicMax on the BF16 magnitude bits (exact, independent of order).
//  * k_select_channels: the k largest channels (ties to the lower index) as a
//    bit mask, and their FP8 scales amax / 448.
//  * k_quant_row_retain: the row-axis fake quantizer's chunk mapping (8
//    elements per lane, blocks and the 128-element outer block by DPP), with
//    the retained columns masked out of every FP4 maximum and encoded to FP8
//    E4M3 under their channel scale.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fq_device.hpp"
#include "fq_internal.h"

using namespace fqdev;

namespace {

constexpr int kThreads = 256;
constexpr uint32_t kGridCap = 1u << 20;

uint32_t grid_for(uint64_t units)
{
    uint64_t g = (units + kThreads - 1) / kThreads;
    if (g > kGridCap) g = kGridCap;
    return (uint32_t)(g ? g : 1);
}

// Streaming accesses: every array of the tracker is read once and written
// once per call and not touched again until the next training step.
typedef float f32v4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32v2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float4 ld_nt(const float4 *p)
{
    const f32v4 v = __builtin_nontemporal_load(reinterpret_cast<const f32v4 *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_nt(const uint2 *p)
{
    const u32v2 v = __builtin_nontemporal_load(reinterpret_cast<const u32v2 *>(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void st_nt(float4 *p, const float4 &v)
{
    __builtin_nontemporal_store((f32v4){v.x, v.y, v.z, v.w}, reinterpret_cast<f32v4 *>(p));
}
__device__ __forceinline__ void st_nt(uint2 *p, const uint2 &v)
{
    __builtin_nontemporal_store((u32v2){v.x, v.y}, reinterpret_cast<u32v2 *>(p));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return as_f(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return as_f(w & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// OsciReset
// ---------------------------------------------------------------------------
// One training step: dist_m += |w - w_prev|, dist_q += |q - q_prev| (FP32,
// each operation rounded once), then w_prev = w, q_prev = q; first = 1 only
// records w and q and clears the distances.
__global__ __launch_bounds__(kThreads) void k_osci_track(const float4 *__restrict__ w,
                                                         const uint2 *__restrict__ q,
                                                         float4 *__restrict__ w_prev,
                                                         uint2 *__restrict__ q_prev,
                                                         float4 *__restrict__ dm,
                                                         float4 *__restrict__ dq, uint64_t n4,
                                                         int first)
{
    // 64-bit index: n4 reaches 2^32 at the largest accepted size
    for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < n4;
         i += (uint64_t)gridDim.x * kThreads) {
        const float4 wv = ld_nt(&w[i]);
        const uint2 qv = ld_nt(&q[i]);
        if (first) {
            st_nt(&dm[i], make_float4(0.0f, 0.0f, 0.0f, 0.0f));
            st_nt(&dq[i], make_float4(0.0f, 0.0f, 0.0f, 0.0f));
        } else {
            const float4 wp = ld_nt(&w_prev[i]);
            const uint2 qp = ld_nt(&q_prev[i]);
            float4 m = ld_nt(&dm[i]), d = ld_nt(&dq[i]);
            m.x = m.x + __builtin_fabsf(wv.x - wp.x);
            m.y = m.y + __builtin_fabsf(wv.y - wp.y);
            m.z = m.z + __builtin_fabsf(wv.z - wp.z);
            m.w = m.w + __builtin_fabsf(wv.w - wp.w);
            d.x = d.x + __builtin_fabsf(bf16_lo(qv.x) - bf16_lo(qp.x));
            d.y = d.y + __builtin_fabsf(bf16_hi(qv.x) - bf16_hi(qp.x));
            d.z = d.z + __builtin_fabsf(bf16_lo(qv.y) - bf16_lo(qp.y));
            d.w = d.w + __builtin_fabsf(bf16_hi(qv.y) - bf16_hi(qp.y));
            st_nt(&dm[i], m);
            st_nt(&dq[i], d);
        }
        st_nt(&w_prev[i], wv);
        st_nt(&q_prev[i], qv);
    }
}

// The check: an element whose dist_q exceeds RN(tau * dist_m) is reset;
// then every element starts a new window (distances 0, trajectory continuing
// from the possibly reset w).
//
// Reset targets:
//  * kTargetCentre (the page's mechanism): the centre of the element's current
//    quantization bin, sign(code) * RN(c_m * s_eff), where c_m is the centre of
//    the interval of scaled magnitudes that round to E2M1 magnitude m:
//    0, 0.5, 1, 1.5, 2.125, 3, 4.25 and 6 (the bins of 2 and 4 are lopsided on
//    the E2M1 grid, [1.75, 2.5] and [3.5, 5]; the top bin is closed at 7, the
//    midpoint with 8, which the format's exponent progression would put next).
//    Code and block scale come from the quantizer outputs that produced q.
//  * kTargetGrid: the quantized value q itself.
enum { kTargetCentre = 0, kTargetGrid = 1 };

// 8 * c_m for m = 0..7 as bytes: {0, 4, 8, 12} and {17, 24, 34, 48}
constexpr uint32_t kCentreLo = 0x0C080400u, kCentreHi = 0x30221811u;

__device__ __forceinline__ float bin_centre(uint32_t code, float s_eff)
{
    const uint32_t m = code & 7u;
    const uint32_t e8 = ((m < 4 ? kCentreLo : kCentreHi) >> (8 * (m & 3))) & 0xFFu;
    const float mag = ((float)e8 * 0.125f) * s_eff;          // c_m exact; one rounding
    return as_f(as_u(mag) | ((code & 8u) << 28));
}

struct OsciQuant {
    const uint8_t *codes;    // E2M1 codes in the quantizer's layout
    const uint8_t *scales;   // block scales in the quantizer's layout
    const float *outer;      // NVFP4 outer scale(s), or null
    uint32_t C;              // columns of w (row-major [R, C])
    uint64_t R;
};

// Code and effective scale of element (r, c) of w from the quantizer outputs:
// row axis codes [R, C/2], scales [R, C/B], outer [R, C/128]; column axis the
// transposed layouts [C, R/2], [C, R/B], [C, R/128].
template <int FMT, bool COL>
__device__ __forceinline__ float centre_of(const OsciQuant &oq, uint64_t r, uint64_t c)
{
    constexpr uint32_t B = FMT == FMT_MX ? 32 : 16;
    const uint64_t qr = COL ? c : r, qc = COL ? r : c;      // quantized orientation
    const uint64_t L = COL ? oq.R : oq.C;                   // its row length
    const uint64_t n = qr * L + qc;
    const uint32_t code = (oq.codes[n >> 1] >> (4 * (uint32_t)(n & 1))) & 0xFu;
    const uint32_t sc = oq.scales[n / B];
    float s_eff;
    if (FMT == FMT_MX) s_eff = e8m0_value(sc);
    else s_eff = e4m3_value(sc) * (FMT == FMT_NVT ? oq.outer[0] : oq.outer[n >> 7]);
    return bin_centre(code, s_eff);
}

template <int TARGET, int FMT, bool COL>
__global__ __launch_bounds__(kThreads) void k_osci_reset(float4 *__restrict__ w,
                                                         const uint2 *__restrict__ q,
                                                         float4 *__restrict__ w_prev,
                                                         uint2 *__restrict__ q_prev,
                                                         float4 *__restrict__ dm,
                                                         float4 *__restrict__ dq, uint64_t n4,
                                                         float tau, OsciQuant oq)
{
    // 64-bit index: n4 reaches 2^32 at the largest accepted size
    for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < n4;
         i += (uint64_t)gridDim.x * kThreads) {
        float4 wv = ld_nt(&w[i]);
        const uint2 qv = ld_nt(&q[i]);
        const float4 m = ld_nt(&dm[i]), d = ld_nt(&dq[i]);
        const bool o0 = d.x > tau * m.x, o1 = d.y > tau * m.y;
        const bool o2 = d.z > tau * m.z, o3 = d.w > tau * m.w;
        if (TARGET == kTargetGrid) {
            wv.x = o0 ? bf16_lo(qv.x) : wv.x;
            wv.y = o1 ? bf16_hi(qv.x) : wv.y;
            wv.z = o2 ? bf16_lo(qv.y) : wv.z;
            wv.w = o3 ? bf16_hi(qv.y) : wv.w;
        } else if (o0 | o1 | o2 | o3) {
            // the four elements 4i .. 4i + 3 share one row (C % 4 == 0); the
            // quantizer outputs are read only for lanes that reset something
            const uint64_t e = 4 * i, r = e / oq.C, c = e % oq.C;
            if (o0) wv.x = centre_of<FMT, COL>(oq, r, c);
            if (o1) wv.y = centre_of<FMT, COL>(oq, r, c + 1);
            if (o2) wv.z = centre_of<FMT, COL>(oq, r, c + 2);
            if (o3) wv.w = centre_of<FMT, COL>(oq, r, c + 3);
        }
        st_nt(&w[i], wv);
        st_nt(&w_prev[i], wv);
        st_nt(&q_prev[i], qv);
        st_nt(&dm[i], make_float4(0.0f, 0.0f, 0.0f, 0.0f));
        st_nt(&dq[i], make_float4(0.0f, 0.0f, 0.0f, 0.0f));
    }
}

// ---------------------------------------------------------------------------
// Outlier channels
// ---------------------------------------------------------------------------
constexpr uint32_t kAmaxRows = 64;     // rows per thread

// Thread t: 8-column chunk t mod (C/8) of rows (t / (C/8)) * 64 .. + 63.
__global__ __launch_bounds__(kThreads) void k_channel_absmax(const uint4 *__restrict__ x,
                                                             uint32_t R, uint32_t C,
                                                             uint32_t *__restrict__ amax)
{
    const uint32_t nchunk = C >> 3;
    const uint64_t t = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    const uint32_t chunk = (uint32_t)(t % nchunk);
    const uint64_t r0 = (t / nchunk) * kAmaxRows;
    if (r0 >= R) return;
    const uint32_t r1 = (uint32_t)min<uint64_t>(r0 + kAmaxRows, R);
    uint32_t m[4] = {0u, 0u, 0u, 0u};
    for (uint32_t r = (uint32_t)r0; r < r1; ++r) {
        const uint4 v = x[(size_t)r * nchunk + chunk];
        m[0] = pkmax_u16(m[0], v.x & 0x7FFF7FFFu);
        m[1] = pkmax_u16(m[1], v.y & 0x7FFF7FFFu);
        m[2] = pkmax_u16(m[2], v.z & 0x7FFF7FFFu);
        m[3] = pkmax_u16(m[3], v.w & 0x7FFF7FFFu);
    }
    uint32_t *dst = amax + (size_t)chunk * 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        atomicMax(&dst[2 * j], m[j] & 0xFFFFu);
        atomicMax(&dst[2 * j + 1], m[j] >> 16);
    }
}

// Thread c: the rank of channel c among all (larger magnitude first, the
// lower index first among equals); retained when rank < k.  The magnitudes
// pass through LDS in tiles of 1024.
constexpr uint32_t kSelTile = 1024;

__global__ __launch_bounds__(kThreads) void k_select_channels(const uint32_t *__restrict__ amax,
                                                              uint32_t C, uint32_t k,
                                                              uint8_t *__restrict__ retain,
                                                              float *__restrict__ chan_scale)
{
    __shared__ uint32_t s_a[kSelTile];
    const uint32_t c = blockIdx.x * kThreads + threadIdx.x;
    const uint32_t mine = c < C ? amax[c] : 0u;
    uint32_t rank = 0;
    for (uint32_t base = 0; base < C; base += kSelTile) {
        const uint32_t nt = min(kSelTile, C - base);
        __syncthreads();
        for (uint32_t i = threadIdx.x; i < nt; i += kThreads) s_a[i] = amax[base + i];
        __syncthreads();
        for (uint32_t i = 0; i < nt; ++i) {
            const uint32_t o = s_a[i];
            rank += (o > mine || (o == mine && base + i < c)) ? 1u : 0u;
        }
    }
    const bool keep = c < C && rank < k;
    if (c < C) chan_scale[c] = keep ? as_f(mine << 16) / 448.0f : 0.0f;
    // bits of 64 consecutive channels -> 8 bytes, written by lane 0
    const uint64_t bits = __ballot(keep);
    const uint32_t c0 = c & ~63u;
    if ((threadIdx.x & 63) == 0 && c0 < C) {
        const uint32_t nbytes = min(8u, (C - c0) / 8);
        for (uint32_t j = 0; j < nbytes; ++j) retain[c0 / 8 + j] = (uint8_t)(bits >> (8 * j));
    }
}

// ---------------------------------------------------------------------------
// Row fake quantization with retained (FP8) channels
// ---------------------------------------------------------------------------
// One 8-element chunk per lane, as the row quantizer's chunk mapping; a
// workgroup covers 256 consecutive chunks of kRetainRows consecutive rows
// (row group and part from the workgroup index, so no per-lane division),
// which also gives every lane its channels directly: chunk j of a row holds
// columns 8j .. 8j + 7, retain byte j, channel scales 8j .. 8j + 7 (two
// 16-byte loads).  The lane sets up the correctly rounded quotient by each of
// its eight channel scales once (reciprocal, and the 2^64 pre-scaling of
// tiny scales, exactly as for an NVFP4 block scale) and reuses it for all
// rows of its group.
constexpr uint32_t kRetainRows = 8;

typedef uint32_t u32v4 __attribute__((ext_vector_type(4)));
// non-temporal load of an input read exactly once
__device__ __forceinline__ uint4 ld_stream(const uint4 *p)
{
    const u32v4 v = __builtin_nontemporal_load(reinterpret_cast<const u32v4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// The per-tensor format reduces the partial maxima of the masked maximum pass
// (retained channels left out) at the start; keep, if given, receives the STE
// keep bits of each chunk (the FP8 test a <= 448 for retained elements).
template <int FMT, int RND, bool NT>
__global__ __launch_bounds__(kThreads) void k_quant_row_retain(
    const uint4 *__restrict__ x, uint32_t R, uint32_t cpr, uint32_t wpr,
    const uint8_t *__restrict__ retain, const float4 *__restrict__ chan_scale,
    uint4 *__restrict__ y, uint32_t *__restrict__ codes, uint8_t *__restrict__ scales,
    float *__restrict__ outer, uint8_t *__restrict__ keep, const uint32_t *__restrict__ partials,
    uint32_t npart, uint32_t seed_lo, uint32_t seed_hi)
{
    OuterScale ot = {0.0f, 0.0f};
    if (FMT == FMT_NVT) {
        ot = tensor_scale<kThreads>(partials, npart);
        if (outer && blockIdx.x == 0 && threadIdx.x == 0) outer[0] = ot.s;
    }
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t group = blockIdx.x / wpr, part = blockIdx.x % wpr;
    const uint32_t j = part * kThreads + threadIdx.x;       // chunk within the row
    if (j >= cpr) return;      // block groups never straddle this edge (C % B == 0)
                               // (after the workgroup-wide per-tensor reduction)
    const uint32_t rbits = retain[j];                       // bit e: element e is an FP8 channel
    BlockScale ch[8];
    if (rbits) {
        const float4 cs0 = chan_scale[2 * j], cs1 = chan_scale[2 * j + 1];
        const float sc[8] = {cs0.x, cs0.y, cs0.z, cs0.w, cs1.x, cs1.y, cs1.z, cs1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ch[e].s_eff = sc[e];
            ch[e].code = 0;
            finish_nv_scale(ch[e]);
        }
    }
    // the FP4 maxima skip the retained elements
    uint32_t fp4m[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        fp4m[i] = (((rbits >> (2 * i)) & 1u) ? 0u : 0x7FFFu) |
                  (((rbits >> (2 * i + 1)) & 1u) ? 0u : 0x7FFF0000u);
    // the retained elements' code nibbles and BF16 halves
    uint32_t nib = 0, sel[4];
#pragma unroll
    for (int e = 0; e < 8; ++e) nib |= ((rbits >> e) & 1u) * (0xFu << (4 * e));
#pragma unroll
    for (int i = 0; i < 4; ++i)
        sel[i] = (((rbits >> (2 * i)) & 1u) ? 0xFFFFu : 0u) |
                 (((rbits >> (2 * i + 1)) & 1u) ? 0xFFFF0000u : 0u);

    // every row's load first, so that all of them are in flight together
    // (streaming: x is read once; rows past the end re-read the last row and
    // are not encoded): 89 -> 79 us for SR, 71 -> 70 us for RNE on 16384x4096
    uint4 xv[kRetainRows];
#pragma unroll
    for (uint32_t r = 0; r < kRetainRows; ++r)
        xv[r] = ld_stream(&x[(size_t)min(group * kRetainRows + r, R - 1) * cpr + j]);
    // every lane of a workgroup has the same row group: the exit is uniform
#pragma unroll
    for (uint32_t r = 0; r < kRetainRows; ++r) {
        const uint32_t row = group * kRetainRows + r;
        if (row >= R) break;
        const size_t c = (size_t)row * cpr + j;
        const uint4 v = xv[r];
        const uint32_t xp[4] = {v.x, v.y, v.z, v.w};
        uint32_t mp[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) mp[i] = xp[i] & fp4m[i];
        const uint32_t m = pkmax_u16(pkmax_u16(mp[0], mp[1]), pkmax_u16(mp[2], mp[3]));
        float so = 0.0f;
        const BlockScale b = chunk_block_scale<FMT>(max(m & 0xFFFFu, m >> 16), ot, so);
        if (FMT == FMT_NV128 && outer && (lane & 15) == 0) outer[c >> 4] = so;
        if (scales) {
            if (FMT == FMT_MX) {
                if ((lane & 3) == 0) scales[c >> 2] = (uint8_t)b.code;
            } else {
                if ((lane & 1) == 0) scales[c >> 1] = (uint8_t)b.code;
            }
        }
        u32x4 rnd[1];
        if (RND == RND_SR)
            rnd[0] = philox4x32_10((uint32_t)c, (uint32_t)(c >> 32), 0u, 0u, seed_lo, seed_hi);
        uint32_t cw[1], yp[4];
        encode_pairs<FMT, RND, 4>(xp, b, rnd, cw, yp);
        uint32_t kb = keep ? keep_mask<FMT, 4>(xp, b) : 0u;
        if (rbits) {
            // every element's FP8 value, then a select per element
            cw[0] &= ~nib;
            uint32_t kr = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bool c0, c1;
                const uint32_t f = fp8_fake_pair(xp[i], ch[2 * i], ch[2 * i + 1], &c0, &c1);
                yp[i] = (f & sel[i]) | (yp[i] & ~sel[i]);
                kr |= (c0 ? 0u : 1u) << (2 * i) | (c1 ? 0u : 1u) << (2 * i + 1);
            }
            kb = (kb & ~rbits) | (kr & rbits);
        }
        if (keep) keep[c] = (uint8_t)kb;
        if (codes) {
            if (NT) __builtin_nontemporal_store(cw[0], &codes[c]);
            else codes[c] = cw[0];
        }
        if (y) {
            const u32v4 o = {yp[0], yp[1], yp[2], yp[3]};
            if (NT) __builtin_nontemporal_store(o, reinterpret_cast<u32v4 *>(&y[c]));
            else *reinterpret_cast<u32v4 *>(&y[c]) = o;
        }
    }
}

template <int FMT, int RND>
hipError_t retain_dispatch(const fqimpl::RetainArgs &a, hipStream_t st)
{
    const uint32_t cpr = (uint32_t)(a.C / 8);
    const uint32_t wpr = (cpr + kThreads - 1) / kThreads;
    const uint64_t groups = ((uint64_t)a.R + kRetainRows - 1) / kRetainRows;
    const uint64_t grid = groups * wpr;
    const uint32_t slo = (uint32_t)a.seed, shi = (uint32_t)(a.seed >> 32);
#define FQ_RETAIN_ARGS                                                                         \
    dim3((uint32_t)grid), dim3(kThreads), 0, st, (const uint4 *)a.x, (uint32_t)a.R, cpr, wpr, \
        (const uint8_t *)a.retain, (const float4 *)a.chan_scale, (uint4 *)a.y,               \
        (uint32_t *)a.codes, (uint8_t *)a.scales, a.outer, (uint8_t *)a.keep, a.partials,      \
        a.npart, slo, shi
    if (a.cached_outputs)
        hipLaunchKernelGGL((k_quant_row_retain<FMT, RND, false>), FQ_RETAIN_ARGS);
    else
        hipLaunchKernelGGL((k_quant_row_retain<FMT, RND, true>), FQ_RETAIN_ARGS);
#undef FQ_RETAIN_ARGS
    return hipGetLastError();
}

}  // namespace

namespace fqimpl {

hipError_t launch_osci_track(const float *w, const void *q, float *w_prev, void *q_prev,
                             float *dist_m, float *dist_q, int64_t n, int first,
                             hipStream_t st)
{
    const uint64_t n4 = (uint64_t)n / 4;
    hipLaunchKernelGGL(k_osci_track, dim3(grid_for(n4)), dim3(kThreads), 0, st,
                       (const float4 *)w, (const uint2 *)q, (float4 *)w_prev, (uint2 *)q_prev,
                       (float4 *)dist_m, (float4 *)dist_q, n4, first);
    return hipGetLastError();
}

hipError_t launch_osci_reset(const OsciResetArgs &a, hipStream_t st)
{
    const uint64_t n4 = (uint64_t)a.n / 4;
    const OsciQuant oq = {(const uint8_t *)a.codes, (const uint8_t *)a.scales, a.outer,
                          (uint32_t)a.C, (uint64_t)a.R};
#define FQ_OSCI_ARGS                                                                        \
    dim3(grid_for(n4)), dim3(kThreads), 0, st, (float4 *)a.w, (const uint2 *)a.q,          \
        (float4 *)a.w_prev, (uint2 *)a.q_prev, (float4 *)a.dist_m, (float4 *)a.dist_q, n4, \
        a.tau, oq
    if (a.grid_target) {
        hipLaunchKernelGGL((k_osci_reset<kTargetGrid, FMT_MX, false>), FQ_OSCI_ARGS);
        return hipGetLastError();
    }
    switch (a.fmt * 2 + (a.col ? 1 : 0)) {
    case FMT_MX * 2 + 0: hipLaunchKernelGGL((k_osci_reset<kTargetCentre, FMT_MX, false>), FQ_OSCI_ARGS); break;
    case FMT_MX * 2 + 1: hipLaunchKernelGGL((k_osci_reset<kTargetCentre, FMT_MX, true>), FQ_OSCI_ARGS); break;
    case FMT_NVT * 2 + 0: hipLaunchKernelGGL((k_osci_reset<kTargetCentre, FMT_NVT, false>), FQ_OSCI_ARGS); break;
    case FMT_NVT * 2 + 1: hipLaunchKernelGGL((k_osci_reset<kTargetCentre, FMT_NVT, true>), FQ_OSCI_ARGS); break;
    case FMT_NV128 * 2 + 0: hipLaunchKernelGGL((k_osci_reset<kTargetCentre, FMT_NV128, false>), FQ_OSCI_ARGS); break;
    case FMT_NV128 * 2 + 1: hipLaunchKernelGGL((k_osci_reset<kTargetCentre, FMT_NV128, true>), FQ_OSCI_ARGS); break;
    default: return hipErrorInvalidValue;
    }
#undef FQ_OSCI_ARGS
    return hipGetLastError();
}

hipError_t launch_channel_absmax(const void *x, int64_t R, int64_t C, uint32_t *amax,
                                 hipStream_t st)
{
    const uint64_t threads = (uint64_t)(C / 8) * (uint64_t)((R + kAmaxRows - 1) / kAmaxRows);
    const uint64_t g = (threads + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(k_channel_absmax, dim3((uint32_t)g), dim3(kThreads), 0, st,
                       (const uint4 *)x, (uint32_t)R, (uint32_t)C, amax);
    return hipGetLastError();
}

hipError_t launch_select_channels(const uint32_t *amax, int64_t C, int64_t k, void *retain,
                                  float *chan_scale, hipStream_t st)
{
    const uint32_t g = (uint32_t)((C + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(k_select_channels, dim3(g), dim3(kThreads), 0, st, amax, (uint32_t)C,
                       (uint32_t)k, (uint8_t *)retain, chan_scale);
    return hipGetLastError();
}

hipError_t launch_quant_retain(const RetainArgs &a, hipStream_t st)
{
    switch (a.fmt * 2 + a.sr) {
    case FMT_MX * 2 + 0: return retain_dispatch<FMT_MX, RND_RNE>(a, st);
    case FMT_MX * 2 + 1: return retain_dispatch<FMT_MX, RND_SR>(a, st);
    case FMT_NVT * 2 + 0: return retain_dispatch<FMT_NVT, RND_RNE>(a, st);
    case FMT_NVT * 2 + 1: return retain_dispatch<FMT_NVT, RND_SR>(a, st);
    case FMT_NV128 * 2 + 0: return retain_dispatch<FMT_NV128, RND_RNE>(a, st);
    case FMT_NV128 * 2 + 1: return retain_dispatch<FMT_NV128, RND_SR>(a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace fqimpl
