// fq_kernels.hip -- streaming FP4 quantize / dequantize / STE kernels, gfx950.
//
// All kernels are HBM-bound streams.  Work is mapped so that every global
// access is a 16-byte vector access coalesced across the wavefront:
//
//  * Row axis (groups along the contiguous dimension): the tensor is a flat
//    array of 8-element chunks (16 bytes of BF16).  Lane i of a wave owns
//    chunk base+i, so a 16-element NVFP4 block is a lane pair, a 32-element
//    MXFP4 block a lane quad, and a 128-element outer block a DPP row of 16
//    lanes.  Block maxima are combined across lanes with DPP, without LDS.
//  * Column axis (groups of B consecutive rows of one column, i.e. the rows
//    of x^T): each lane owns an 8-column x B-row tile and loads it as B
//    row segments of 16 bytes.  The 64 lanes of a wave cover 64 columns x
//    8 row blocks; for one column the 8 lanes of consecutive row blocks
//    write adjacent code bytes, so transposed codes leave the wave as
//    contiguous 64-byte (NVFP4) or 128-byte (MXFP4) runs.  The 128-row outer
//    block of the double-block format is those 8 lanes (DPP half-row).
//
// Numerics follow fq_device.hpp; the op definitions are those of fq.h.
#include "fq_device.hpp"
#include "fq_internal.h"

using namespace fqdev;

namespace {

constexpr int kThreads = 256;
constexpr uint32_t kRowGridCap = 4096;   // workgroups for grid-stride streams

// ---------------------------------------------------------------------------
// Per-tensor maximum: partial maxima of |x| (as BF16 magnitude bits), one per
// workgroup.  Consumers reduce the partials themselves, so no zero-filled
// accumulator and no atomics are needed.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t block_reduce_max(uint32_t m, uint32_t *red)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        m = max(m, (uint32_t)__shfl_xor((int)m, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    return m;
}

__global__ __launch_bounds__(kThreads) void k_absmax(const uint4 *__restrict__ x,
                                                     uint32_t nchunks,
                                                     uint32_t *__restrict__ partials)
{
    __shared__ uint32_t red[4];
    uint32_t m = 0;
    const uint32_t stride = gridDim.x * kThreads * 4;
    for (uint32_t base = blockIdx.x * kThreads * 4; base < nchunks; base += stride) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            uint32_t c = base + u * kThreads + threadIdx.x;
            v[u] = c < nchunks ? x[c] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) m = max(m, absmax_bits_8(v[u]));
    }
    m = block_reduce_max(m, red);
    if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// NVFP4 per-tensor outer scale from the partial maxima (every thread).
__device__ __forceinline__ float tensor_scale(const uint32_t *__restrict__ partials,
                                              uint32_t npart)
{
    __shared__ uint32_t red[4];
    uint32_t m = 0;
    for (uint32_t i = threadIdx.x; i < npart; i += kThreads) m = max(m, partials[i]);
    m = block_reduce_max(m, red);
    return nv_outer_scale(as_f(m << 16));
}

// Block scale rebuilt from a stored scale code (dequantize, STE).
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

// Encode one element: returns the 4-bit code and the signed FP32 value
// g * s_eff (before BF16 rounding).
template <int FMT, int RND>
__device__ __forceinline__ uint32_t encode_elem(uint32_t xb, const BlockScale &b,
                                                uint32_t r16, float &yv)
{
    float a = scaled_mag<FMT>(xb, b);
    uint32_t m;
    float g;
    if (RND == RND_RNE) {
        e2m1_rne(a, m, g);
    } else {
        m = e2m1_sr(a, r16);
        g = e2m1_value(m);
    }
    yv = as_f(as_u(g * b.s_eff) | (xb & 0x80000000u));
    return m | ((xb >> 28) & 8u);
}

// ---------------------------------------------------------------------------
// Row-axis quantizer (flat chunk stream)
// ---------------------------------------------------------------------------
template <int FMT, int RND>
__device__ __forceinline__ void quant_row_chunk(uint32_t c, const uint4 &v, float s_t,
                                                uint4 *__restrict__ y,
                                                uint32_t *__restrict__ codes,
                                                uint8_t *__restrict__ scales,
                                                float *__restrict__ outer,
                                                uint32_t seed_lo, uint32_t seed_hi)
{
    const uint32_t lane = threadIdx.x & 63;
    uint32_t mb = dpp_max_xor1(absmax_bits_8(v));
    BlockScale b;
    if (FMT == FMT_MX) {
        mb = dpp_max_xor2(mb);
        b = mx_block_scale(mb);
    } else {
        float s = s_t;
        if (FMT == FMT_NV128) {
            uint32_t mo = dpp_max_ror8(dpp_max_ror4(dpp_max_xor2(mb)));
            s = nv_outer_scale(as_f(mo << 16));
            if (outer && (lane & 15) == 0) outer[c >> 4] = s;
        }
        b = nv_block_scale(as_f(mb << 16), s);
    }
    if (scales) {
        if (FMT == FMT_MX) {
            if ((lane & 3) == 0) scales[c >> 2] = (uint8_t)b.code;
        } else {
            if ((lane & 1) == 0) scales[c >> 1] = (uint8_t)b.code;
        }
    }
    u32x4 rnd;
    if (RND == RND_SR) rnd = philox4x32_10(c, 0u, 0u, 0u, seed_lo, seed_hi);
    uint32_t packed = 0;
    float yv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t r16 = 0;
        if (RND == RND_SR) r16 = (rnd.v[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
        uint32_t code = encode_elem<FMT, RND>(elem_bits(v, j), b, r16, yv[j]);
        packed |= code << (4 * j);
    }
    if (codes) codes[c] = packed;
    if (y) {
        y[c] = make_uint4(bf16_pair_rne(yv[0], yv[1]), bf16_pair_rne(yv[2], yv[3]),
                          bf16_pair_rne(yv[4], yv[5]), bf16_pair_rne(yv[6], yv[7]));
    }
}

template <int FMT, int RND>
__global__ __launch_bounds__(kThreads) void k_quant_row(
    const uint4 *__restrict__ x, uint32_t nchunks, uint4 *__restrict__ y,
    uint32_t *__restrict__ codes, uint8_t *__restrict__ scales, float *__restrict__ outer,
    const uint32_t *__restrict__ partials, uint32_t npart, uint32_t seed_lo,
    uint32_t seed_hi)
{
    float s_t = 0.0f;
    if (FMT == FMT_NVT) {
        s_t = tensor_scale(partials, npart);
        if (outer && blockIdx.x == 0 && threadIdx.x == 0) outer[0] = s_t;
    }
    const uint32_t stride = gridDim.x * kThreads * 2;
    for (uint32_t base = blockIdx.x * kThreads * 2; base < nchunks; base += stride) {
        const uint32_t c0 = base + threadIdx.x, c1 = c0 + kThreads;
        uint4 v0 = make_uint4(0, 0, 0, 0), v1 = make_uint4(0, 0, 0, 0);
        if (c0 < nchunks) v0 = x[c0];
        if (c1 < nchunks) v1 = x[c1];
        if (c0 < nchunks)
            quant_row_chunk<FMT, RND>(c0, v0, s_t, y, codes, scales, outer, seed_lo, seed_hi);
        if (c1 < nchunks)
            quant_row_chunk<FMT, RND>(c1, v1, s_t, y, codes, scales, outer, seed_lo, seed_hi);
    }
}

// ---------------------------------------------------------------------------
// Column-axis quantizer (lane = 8 columns x B rows)
// ---------------------------------------------------------------------------
// BF16 half-word c (0..7) of a 16-byte row segment, as FP32 bits.
__device__ __forceinline__ uint32_t seg_elem(const uint4 &v, int c) { return elem_bits(v, c); }

__device__ __forceinline__ void seg_set_pair(uint4 &v, int p, uint32_t w)
{
    if (p == 0) v.x = w;
    else if (p == 1) v.y = w;
    else if (p == 2) v.z = w;
    else v.w = w;
}

template <int FMT, int RND>
__global__ __launch_bounds__(kThreads) void k_quant_col(
    const uint4 *__restrict__ x, uint32_t R, uint32_t C, uint4 *__restrict__ y,
    uint4 *__restrict__ yt, uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
    float *__restrict__ outer, const uint32_t *__restrict__ partials, uint32_t npart,
    uint32_t seed_lo, uint32_t seed_hi)
{
    constexpr int B = (FMT == FMT_MX) ? 32 : 16;
    float s_t = 0.0f;
    if (FMT == FMT_NVT) {
        s_t = tensor_scale(partials, npart);
        if (outer && blockIdx.x == 0 && threadIdx.x == 0) outer[0] = s_t;
    }
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t rb = lane & 7, cg = lane >> 3;
    const uint32_t tiles_c = (C + 63) >> 6;           // 1-D grid: column tiles fastest
    const uint32_t col0 = (blockIdx.x % tiles_c) * 64 + cg * 8;
    const uint32_t row0 = (((blockIdx.x / tiles_c) * 4 + wave) * 8 + rb) * B;
    if (col0 >= C || row0 >= R) return;   // whole 8-lane groups leave together for NV128
    const uint32_t ldx = C >> 3;            // 16-byte segments per row

    uint4 v[B];
#pragma unroll
    for (int r = 0; r < B; ++r) v[r] = x[(size_t)(row0 + r) * ldx + (col0 >> 3)];

    // per-column block maxima: packed u16 max over the B rows
    uint32_t mw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int r = 0; r < B; ++r) {
        mw[0] = pkmax_u16(mw[0], v[r].x & 0x7FFF7FFFu);
        mw[1] = pkmax_u16(mw[1], v[r].y & 0x7FFF7FFFu);
        mw[2] = pkmax_u16(mw[2], v[r].z & 0x7FFF7FFFu);
        mw[3] = pkmax_u16(mw[3], v[r].w & 0x7FFF7FFFu);
    }

#pragma unroll
    for (int p = 0; p < 4; ++p) {
        BlockScale bs[2];
        u32x4 rnd[2][B / 8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t col = col0 + 2 * p + h;
            uint32_t m = h ? (mw[p] >> 16) : (mw[p] & 0xFFFFu);
            if (FMT == FMT_MX) {
                bs[h] = mx_block_scale(m);
            } else {
                float s = s_t;
                if (FMT == FMT_NV128) {
                    uint32_t mo = dpp_max_half_mirror(dpp_max_xor2(dpp_max_xor1(m)));
                    s = nv_outer_scale(as_f(mo << 16));
                    if (outer && (rb & 7) == 0)
                        outer[(size_t)col * (R >> 7) + (row0 >> 7)] = s;
                }
                bs[h] = nv_block_scale(as_f(m << 16), s);
            }
            if (scales) scales[(size_t)col * (R / B) + row0 / B] = (uint8_t)bs[h].code;
            if (RND == RND_SR) {
                const uint64_t call0 = ((uint64_t)col * R + row0) >> 3;
#pragma unroll
                for (int k = 0; k < B / 8; ++k) {
                    const uint64_t cl = call0 + k;
                    rnd[h][k] = philox4x32_10((uint32_t)cl, (uint32_t)(cl >> 32), 0u, 0u,
                                              seed_lo, seed_hi);
                }
            }
        }
        uint32_t cw[2][B / 8];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int k = 0; k < B / 8; ++k) cw[h][k] = 0u;
        uint32_t ytw[2][B / 2];
        float yprev[2] = {0.0f, 0.0f};
#pragma unroll
        for (int r = 0; r < B; ++r) {
            float yv[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t r16 = 0;
                if (RND == RND_SR)
                    r16 = (rnd[h][r >> 3].v[(r >> 1) & 3] >> (16 * (r & 1))) & 0xFFFFu;
                uint32_t code = encode_elem<FMT, RND>(seg_elem(v[r], 2 * p + h), bs[h], r16, yv[h]);
                cw[h][r >> 3] |= code << (4 * (r & 7));
                if (r & 1) ytw[h][r >> 1] = bf16_pair_rne(yprev[h], yv[h]);
                yprev[h] = yv[h];
            }
            seg_set_pair(v[r], p, bf16_pair_rne(yv[0], yv[1]));
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t col = col0 + 2 * p + h;
            if (codes) {
                uint8_t *dst = codes + (size_t)col * (R >> 1) + (row0 >> 1);
                if constexpr (B == 16) {
                    *reinterpret_cast<uint2 *>(dst) = make_uint2(cw[h][0], cw[h][1]);
                } else {
                    *reinterpret_cast<uint4 *>(dst) = make_uint4(cw[h][0], cw[h][1], cw[h][2], cw[h][3]);
                }
            }
            if (yt) {
                uint4 *dst = yt + (((size_t)col * R + row0) >> 3);
#pragma unroll
                for (int k = 0; k < B / 8; ++k)
                    dst[k] = make_uint4(ytw[h][4 * k], ytw[h][4 * k + 1], ytw[h][4 * k + 2],
                                        ytw[h][4 * k + 3]);
            }
        }
    }
    if (y) {
#pragma unroll
        for (int r = 0; r < B; ++r) y[(size_t)(row0 + r) * ldx + (col0 >> 3)] = v[r];
    }
}

// ---------------------------------------------------------------------------
// Dequantize
// ---------------------------------------------------------------------------
__device__ __forceinline__ float decode_elem(uint32_t code, float s_eff)
{
    return as_f(as_u(e2m1_value(code & 7u) * s_eff) | ((code & 8u) << 28));
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_dequant_row(
    const uint32_t *__restrict__ codes, const uint8_t *__restrict__ scales,
    const float *__restrict__ outer, uint32_t nchunks, uint4 *__restrict__ y)
{
    const float s_t = (FMT == FMT_NVT) ? outer[0] : 0.0f;
    for (uint32_t c = blockIdx.x * kThreads + threadIdx.x; c < nchunks;
         c += gridDim.x * kThreads) {
        const uint32_t packed = codes[c];
        float s = s_t;
        if (FMT == FMT_NV128) s = outer[c >> 4];
        const uint32_t sc = scales[FMT == FMT_MX ? (c >> 2) : (c >> 1)];
        const float s_eff = (FMT == FMT_MX) ? e8m0_value(sc) : e4m3_value(sc) * s;
        float yv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) yv[j] = decode_elem((packed >> (4 * j)) & 15u, s_eff);
        y[c] = make_uint4(bf16_pair_rne(yv[0], yv[1]), bf16_pair_rne(yv[2], yv[3]),
                          bf16_pair_rne(yv[4], yv[5]), bf16_pair_rne(yv[6], yv[7]));
    }
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_dequant_col(
    const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
    const float *__restrict__ outer, uint32_t R, uint32_t C, uint4 *__restrict__ y)
{
    constexpr int B = (FMT == FMT_MX) ? 32 : 16;
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t rb = lane & 7, cg = lane >> 3;
    const uint32_t tiles_c = (C + 63) >> 6;           // 1-D grid: column tiles fastest
    const uint32_t col0 = (blockIdx.x % tiles_c) * 64 + cg * 8;
    const uint32_t row0 = (((blockIdx.x / tiles_c) * 4 + wave) * 8 + rb) * B;
    if (col0 >= C || row0 >= R) return;
    const uint32_t ldx = C >> 3;
    uint4 v[B];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        uint32_t cw[2][B / 8];
        float se[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t col = col0 + 2 * p + h;
            const uint8_t *src = codes + (size_t)col * (R >> 1) + (row0 >> 1);
            if constexpr (B == 16) {
                uint2 t = *reinterpret_cast<const uint2 *>(src);
                cw[h][0] = t.x;
                cw[h][1] = t.y;
            } else {
                uint4 t = *reinterpret_cast<const uint4 *>(src);
                cw[h][0] = t.x;
                cw[h][1] = t.y;
                cw[h][2] = t.z;
                cw[h][3] = t.w;
            }
            const uint32_t sc = scales[(size_t)col * (R / B) + row0 / B];
            float s = 0.0f;
            if (FMT == FMT_NVT) s = outer[0];
            if (FMT == FMT_NV128) s = outer[(size_t)col * (R >> 7) + (row0 >> 7)];
            se[h] = (FMT == FMT_MX) ? e8m0_value(sc) : e4m3_value(sc) * s;
        }
#pragma unroll
        for (int r = 0; r < B; ++r) {
            float y0 = decode_elem((cw[0][r >> 3] >> (4 * (r & 7))) & 15u, se[0]);
            float y1 = decode_elem((cw[1][r >> 3] >> (4 * (r & 7))) & 15u, se[1]);
            seg_set_pair(v[r], p, bf16_pair_rne(y0, y1));
        }
    }
#pragma unroll
    for (int r = 0; r < B; ++r) y[(size_t)(row0 + r) * ldx + (col0 >> 3)] = v[r];
}

// ---------------------------------------------------------------------------
// Straight-through estimator with clipping mask
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ste_half(uint32_t dyw, uint32_t keep_lo, uint32_t keep_hi)
{
    return (keep_lo ? (dyw & 0xFFFFu) : 0u) | (keep_hi ? (dyw & 0xFFFF0000u) : 0u);
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_ste_row(
    const uint4 *__restrict__ x, const uint8_t *__restrict__ scales,
    const float *__restrict__ outer, const uint4 *__restrict__ dy, uint32_t nchunks,
    uint4 *__restrict__ dx)
{
    const float s_t = (FMT == FMT_NVT) ? outer[0] : 0.0f;
    for (uint32_t c = blockIdx.x * kThreads + threadIdx.x; c < nchunks;
         c += gridDim.x * kThreads) {
        const uint4 v = x[c];
        const uint4 d = dy[c];
        float s = s_t;
        if (FMT == FMT_NV128) s = outer[c >> 4];
        const BlockScale b =
            scale_from_code<FMT>(scales[FMT == FMT_MX ? (c >> 2) : (c >> 1)], s);
        uint32_t keep[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) keep[j] = scaled_mag<FMT>(elem_bits(v, j), b) <= 6.0f;
        dx[c] = make_uint4(ste_half(d.x, keep[0], keep[1]), ste_half(d.y, keep[2], keep[3]),
                           ste_half(d.z, keep[4], keep[5]), ste_half(d.w, keep[6], keep[7]));
    }
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_ste_col(
    const uint4 *__restrict__ x, const uint8_t *__restrict__ scales,
    const float *__restrict__ outer, const uint4 *__restrict__ dy, uint32_t R, uint32_t C,
    uint4 *__restrict__ dx)
{
    constexpr int B = (FMT == FMT_MX) ? 32 : 16;
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t rb = lane & 7, cg = lane >> 3;
    const uint32_t tiles_c = (C + 63) >> 6;           // 1-D grid: column tiles fastest
    const uint32_t col0 = (blockIdx.x % tiles_c) * 64 + cg * 8;
    const uint32_t row0 = (((blockIdx.x / tiles_c) * 4 + wave) * 8 + rb) * B;
    if (col0 >= C || row0 >= R) return;
    const uint32_t ldx = C >> 3;
    BlockScale bs[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint32_t col = col0 + c;
        float s = 0.0f;
        if (FMT == FMT_NVT) s = outer[0];
        if (FMT == FMT_NV128) s = outer[(size_t)col * (R >> 7) + (row0 >> 7)];
        bs[c] = scale_from_code<FMT>(scales[(size_t)col * (R / B) + row0 / B], s);
    }
#pragma unroll 4
    for (int r = 0; r < B; ++r) {
        const size_t idx = (size_t)(row0 + r) * ldx + (col0 >> 3);
        const uint4 v = x[idx];
        const uint4 d = dy[idx];
        uint32_t keep[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) keep[c] = scaled_mag<FMT>(elem_bits(v, c), bs[c]) <= 6.0f;
        dx[idx] = make_uint4(ste_half(d.x, keep[0], keep[1]), ste_half(d.y, keep[2], keep[3]),
                             ste_half(d.z, keep[4], keep[5]), ste_half(d.w, keep[6], keep[7]));
    }
}

// ---------------------------------------------------------------------------
// launch helpers
// ---------------------------------------------------------------------------
uint32_t row_grid(uint64_t nchunks, uint32_t per_block)
{
    uint64_t g = (nchunks + per_block - 1) / per_block;
    if (g > kRowGridCap) g = kRowGridCap;
    if (g == 0) g = 1;
    return (uint32_t)g;
}

// Column-axis grid: one workgroup per 64-column x (4 waves x 8 blocks) tile.
dim3 col_grid(int64_t R, int64_t C, int B)
{
    uint64_t gx = (uint64_t)((C + 63) / 64);
    uint64_t gy = (uint64_t)((R + 32 * B - 1) / (32 * B));
    return dim3((uint32_t)(gx * gy), 1, 1);
}

template <int FMT, int RND>
hipError_t quant_dispatch(const fqimpl::QuantArgs &a, uint32_t npart, hipStream_t st)
{
    const uint32_t slo = (uint32_t)a.seed, shi = (uint32_t)(a.seed >> 32);
    const uint32_t *parts = a.partials;
    if (!a.col) {
        const uint64_t nchunks = (uint64_t)a.R * a.C / 8;
        hipLaunchKernelGGL((k_quant_row<FMT, RND>), dim3(row_grid(nchunks, kThreads * 2)),
                           dim3(kThreads), 0, st, (const uint4 *)a.x, (uint32_t)nchunks,
                           (uint4 *)a.y, (uint32_t *)a.codes, (uint8_t *)a.scales, a.outer,
                           parts, npart, slo, shi);
    } else {
        const int B = (FMT == FMT_MX) ? 32 : 16;
        hipLaunchKernelGGL((k_quant_col<FMT, RND>), col_grid(a.R, a.C, B), dim3(kThreads), 0,
                           st, (const uint4 *)a.x, (uint32_t)a.R, (uint32_t)a.C, (uint4 *)a.y,
                           (uint4 *)a.yt, (uint8_t *)a.codes, (uint8_t *)a.scales, a.outer, parts, npart,
                           slo, shi);
    }
    return hipGetLastError();
}

}  // namespace

namespace fqimpl {

hipError_t launch_absmax(const void *x, int64_t n_elems, uint32_t *partials,
                         uint32_t *npart_out, hipStream_t stream)
{
    const uint64_t nchunks = (uint64_t)n_elems / 8;
    uint64_t g = (nchunks + kThreads * 4 - 1) / (kThreads * 4);
    if (g > kAbsmaxPartials) g = kAbsmaxPartials;
    if (g == 0) g = 1;
    hipLaunchKernelGGL(k_absmax, dim3((uint32_t)g), dim3(kThreads), 0, stream,
                       (const uint4 *)x, (uint32_t)nchunks, partials);
    *npart_out = (uint32_t)g;
    return hipGetLastError();
}

hipError_t launch_quant(const QuantArgs &a, uint32_t npart, hipStream_t st)
{
    switch (a.fmt * 2 + a.sr) {
    case FMT_MX * 2 + 0: return quant_dispatch<FMT_MX, RND_RNE>(a, npart, st);
    case FMT_MX * 2 + 1: return quant_dispatch<FMT_MX, RND_SR>(a, npart, st);
    case FMT_NVT * 2 + 0: return quant_dispatch<FMT_NVT, RND_RNE>(a, npart, st);
    case FMT_NVT * 2 + 1: return quant_dispatch<FMT_NVT, RND_SR>(a, npart, st);
    case FMT_NV128 * 2 + 0: return quant_dispatch<FMT_NV128, RND_RNE>(a, npart, st);
    case FMT_NV128 * 2 + 1: return quant_dispatch<FMT_NV128, RND_SR>(a, npart, st);
    default: return hipErrorInvalidValue;
    }
}

template <int FMT>
static hipError_t dequant_dispatch(int col, const void *codes, const void *scales,
                                   const float *outer, int64_t R, int64_t C, void *y,
                                   hipStream_t st)
{
    if (!col) {
        const uint64_t nchunks = (uint64_t)R * C / 8;
        hipLaunchKernelGGL(k_dequant_row<FMT>, dim3(row_grid(nchunks, kThreads)),
                           dim3(kThreads), 0, st, (const uint32_t *)codes,
                           (const uint8_t *)scales, outer, (uint32_t)nchunks, (uint4 *)y);
    } else {
        const int B = (FMT == FMT_MX) ? 32 : 16;
        hipLaunchKernelGGL(k_dequant_col<FMT>, col_grid(R, C, B), dim3(kThreads), 0, st,
                           (const uint8_t *)codes, (const uint8_t *)scales, outer,
                           (uint32_t)R, (uint32_t)C, (uint4 *)y);
    }
    return hipGetLastError();
}

hipError_t launch_dequant(int fmt, int col, const void *codes, const void *scales,
                          const float *outer, int64_t R, int64_t C, void *y,
                          hipStream_t stream)
{
    switch (fmt) {
    case FMT_MX: return dequant_dispatch<FMT_MX>(col, codes, scales, outer, R, C, y, stream);
    case FMT_NVT: return dequant_dispatch<FMT_NVT>(col, codes, scales, outer, R, C, y, stream);
    case FMT_NV128:
        return dequant_dispatch<FMT_NV128>(col, codes, scales, outer, R, C, y, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int FMT>
static hipError_t ste_dispatch(int col, const void *x, const void *scales, const float *outer,
                               const void *dy, int64_t R, int64_t C, void *dx, hipStream_t st)
{
    if (!col) {
        const uint64_t nchunks = (uint64_t)R * C / 8;
        hipLaunchKernelGGL(k_ste_row<FMT>, dim3(row_grid(nchunks, kThreads)), dim3(kThreads),
                           0, st, (const uint4 *)x, (const uint8_t *)scales, outer,
                           (const uint4 *)dy, (uint32_t)nchunks, (uint4 *)dx);
    } else {
        const int B = (FMT == FMT_MX) ? 32 : 16;
        hipLaunchKernelGGL(k_ste_col<FMT>, col_grid(R, C, B), dim3(kThreads), 0, st,
                           (const uint4 *)x, (const uint8_t *)scales, outer, (const uint4 *)dy,
                           (uint32_t)R, (uint32_t)C, (uint4 *)dx);
    }
    return hipGetLastError();
}

hipError_t launch_ste(int fmt, int col, const void *x, const void *scales, const float *outer,
                      const void *dy, int64_t R, int64_t C, void *dx, hipStream_t stream)
{
    switch (fmt) {
    case FMT_MX: return ste_dispatch<FMT_MX>(col, x, scales, outer, dy, R, C, dx, stream);
    case FMT_NVT: return ste_dispatch<FMT_NVT>(col, x, scales, outer, dy, R, C, dx, stream);
    case FMT_NV128: return ste_dispatch<FMT_NV128>(col, x, scales, outer, dy, R, C, dx, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace fqimpl
