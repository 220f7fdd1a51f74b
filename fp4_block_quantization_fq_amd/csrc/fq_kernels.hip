// fq_kernels.hip -- streaming FP4 quantize / dequantize / STE kernels, gfx950.
//
// All kernels are HBM-bound streams.  A lane always owns 16 consecutive
// elements along the quantization axis (one NVFP4 block, half an MXFP4 block),
// and every global access is a 16-byte vector access coalesced across the
// wavefront:
//
//  * Row axis (groups along the contiguous dimension): the tensor is a flat
//    array of 16-element segments (32 bytes of BF16).  Lane i of a wave owns
//    segment base+i, so an MXFP4 block is a lane pair and a 128-element outer
//    block is 8 lanes; block maxima are combined with DPP, without LDS.
//  * Column axis (groups of consecutive rows of one column, i.e. the rows of
//    x^T): a lane owns an 8-column x 16-row tile, loaded as 16 row segments
//    of 16 bytes.  The 64 lanes of a wave cover 64 columns x 128 rows; the
//    8 lanes of one column group hold consecutive row blocks, so their
//    transposed code bytes leave the wave as one contiguous 64-byte run per
//    column, MXFP4 blocks are lane pairs and the double-block's 128-row outer
//    block is those 8 lanes.
//
// Numerics follow fq_device.hpp; the op definitions are those of fq.h.
#include "fq_device.hpp"
#include "fq_internal.h"

using namespace fqdev;

namespace {

// Row-axis streams, chosen by measurement on MI355X (16384 x 4096 BF16):
//  - round-to-nearest kernels, the STE and dequantize map one 8-element chunk
//    to a lane (every load and store instruction is one contiguous 1 KB run);
//  - stochastic-rounding kernels, which are bound by Philox and encoder ALU
//    work, map a 16-element segment to a lane, halving the per-lane block
//    scale work;
//  - one unit per thread and a grid as large as the tensor (capped), so that
//    every CU has many waves in flight;
//  - streamed outputs use non-temporal stores (they are not re-read by the
//    kernel, and keeping them out of the caches helps the input stream); the
//    QAT linear writes its operands with ordinary stores because the GEMM
//    reads them right away.
constexpr int kThreads = 256;
constexpr uint32_t kRowGridCap = 1u << 20;

typedef uint32_t u32v4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32v2 __attribute__((ext_vector_type(2)));

template <bool NT>
__device__ __forceinline__ void st_stream(uint4 *p, const uint4 &v)
{
    if (NT) __builtin_nontemporal_store((u32v4){v.x, v.y, v.z, v.w}, reinterpret_cast<u32v4 *>(p));
    else *p = v;
}
template <bool NT>
__device__ __forceinline__ void st_stream(uint2 *p, const uint2 &v)
{
    if (NT) __builtin_nontemporal_store((u32v2){v.x, v.y}, reinterpret_cast<u32v2 *>(p));
    else *p = v;
}
template <bool NT>
__device__ __forceinline__ void st_stream(uint32_t *p, uint32_t v)
{
    if (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// ---------------------------------------------------------------------------
// Per-tensor maximum: partial maxima of |x| (as BF16 magnitude bits), one per
// workgroup.  Consumers reduce the partials themselves, so no zero-filled
// accumulator and no atomics are needed.
// ---------------------------------------------------------------------------
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

// One workgroup of kAbsmaxThreads per partial; at most kAbsmaxGrid partials,
// so that every quantizer workgroup reduces at most 1 KB of them.
constexpr int kAbsmaxThreads = 1024;
constexpr uint32_t kAbsmaxGrid = 256;
static_assert(kAbsmaxGrid <= fqimpl::kAbsmaxPartials, "partials fit the workspace");

__global__ __launch_bounds__(kAbsmaxThreads) void k_absmax(const uint4 *__restrict__ x,
                                                           uint32_t nchunks,
                                                           uint32_t *__restrict__ partials)
{
    __shared__ uint32_t red[kAbsmaxThreads / 64];
    uint32_t m = 0;
    const uint32_t stride = gridDim.x * kAbsmaxThreads * 4;
    for (uint32_t base = blockIdx.x * kAbsmaxThreads * 4; base < nchunks; base += stride) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            uint32_t c = base + u * kAbsmaxThreads + threadIdx.x;
            v[u] = c < nchunks ? x[c] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) m = max(m, absmax_bits_8(v[u]));
    }
    m = block_reduce_max<kAbsmaxThreads>(m, red);
    if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// NVFP4 per-tensor outer scale from the partial maxima (every thread).
__device__ __forceinline__ OuterScale tensor_scale(const uint32_t *__restrict__ partials,
                                                   uint32_t npart)
{
    __shared__ uint32_t red[kThreads / 64];
    uint32_t m = 0;
    for (uint32_t i = threadIdx.x; i < npart; i += kThreads) m = max(m, partials[i]);
    m = block_reduce_max<kThreads>(m, red);
    return make_outer(as_f(m << 16));
}

// Block scale of this lane's 16 elements (cross-lane for MXFP4 and the
// double block).  `outer_out` receives the 128-block outer scale (NV128).
template <int FMT>
__device__ __forceinline__ BlockScale lane_block_scale(uint32_t amax16, const OuterScale &ot,
                                                       float &outer_out)
{
    if (FMT == FMT_MX) return mx_block_scale(dpp_max_xor1(amax16));
    if (FMT == FMT_NVT) return nv_block_scale(as_f(amax16 << 16), ot);
    const uint32_t mo = dpp_max_8lanes(amax16);
    const OuterScale o = make_outer(as_f(mo << 16));
    outer_out = o.s;
    return nv_block_scale(as_f(amax16 << 16), o);
}

// ---------------------------------------------------------------------------
// Row-axis quantizer (flat segment stream)
// ---------------------------------------------------------------------------
template <int FMT, int RND, bool NT>
__device__ __forceinline__ void quant_row_seg(uint32_t seg, const uint4 &v0, const uint4 &v1,
                                              const OuterScale &ot, uint4 *__restrict__ y,
                                              uint2 *__restrict__ codes,
                                              uint8_t *__restrict__ scales,
                                              float *__restrict__ outer, uint32_t seed_lo,
                                              uint32_t seed_hi)
{
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t xp[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    float so = 0.0f;
    const BlockScale b = lane_block_scale<FMT>(absmax_bits_pairs8(xp), ot, so);
    if (FMT == FMT_NV128 && outer && (lane & 7) == 0) outer[seg >> 3] = so;
    if (scales) {
        if (FMT == FMT_MX) {
            if ((lane & 1) == 0) scales[seg >> 1] = (uint8_t)b.code;
        } else {
            scales[seg] = (uint8_t)b.code;
        }
    }
    u32x4 rnd[2];
    if (RND == RND_SR) {
        rnd[0] = philox4x32_10(2 * seg, 0u, 0u, 0u, seed_lo, seed_hi);
        rnd[1] = philox4x32_10(2 * seg + 1, 0u, 0u, 0u, seed_lo, seed_hi);
    }
    uint32_t cw[2], yp[8];
    encode_pairs<FMT, RND, 8>(xp, b, rnd, cw, yp);
    if (codes) st_stream<NT>(&codes[seg], make_uint2(cw[0], cw[1]));
    if (y) {
        st_stream<NT>(&y[2 * seg], make_uint4(yp[0], yp[1], yp[2], yp[3]));
        st_stream<NT>(&y[2 * seg + 1], make_uint4(yp[4], yp[5], yp[6], yp[7]));
    }
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

template <int FMT, int RND, bool NT>
__device__ __forceinline__ void quant_row_chunk(uint32_t c, const uint4 &v, const OuterScale &ot,
                                                uint4 *__restrict__ y,
                                                uint32_t *__restrict__ codes,
                                                uint8_t *__restrict__ scales,
                                                float *__restrict__ outer, uint32_t seed_lo,
                                                uint32_t seed_hi)
{
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t xp[4] = {v.x, v.y, v.z, v.w};
    float so = 0.0f;
    const BlockScale b = chunk_block_scale<FMT>(absmax_bits_8(v), ot, so);
    if (FMT == FMT_NV128 && outer && (lane & 15) == 0) outer[c >> 4] = so;
    if (scales) {
        if (FMT == FMT_MX) {
            if ((lane & 3) == 0) scales[c >> 2] = (uint8_t)b.code;
        } else {
            if ((lane & 1) == 0) scales[c >> 1] = (uint8_t)b.code;
        }
    }
    u32x4 rnd[1];
    if (RND == RND_SR) rnd[0] = philox4x32_10(c, 0u, 0u, 0u, seed_lo, seed_hi);
    uint32_t cw[1], yp[4];
    encode_pairs<FMT, RND, 4>(xp, b, rnd, cw, yp);
    if (codes) st_stream<NT>(&codes[c], cw[0]);
    if (y) st_stream<NT>(&y[c], make_uint4(yp[0], yp[1], yp[2], yp[3]));
}

// MAP = 1: one 8-element chunk per lane (units = chunks); MAP = 0: one
// 16-element segment per lane (units = segments).
template <int FMT, int RND, int MAP, bool NT>
__global__ __launch_bounds__(kThreads) void k_quant_row(
    const uint4 *__restrict__ x, uint32_t nunits, uint4 *__restrict__ y,
    void *__restrict__ codes, uint8_t *__restrict__ scales, float *__restrict__ outer,
    const uint32_t *__restrict__ partials, uint32_t npart, uint32_t seed_lo,
    uint32_t seed_hi)
{
    OuterScale ot = {0.0f, 0.0f};
    if (FMT == FMT_NVT) {
        ot = tensor_scale(partials, npart);
        if (outer && blockIdx.x == 0 && threadIdx.x == 0) outer[0] = ot.s;
    }
    for (uint32_t u = blockIdx.x * kThreads + threadIdx.x; u < nunits;
         u += gridDim.x * kThreads) {
        if (MAP == 1) {
            const uint4 v = x[u];
            quant_row_chunk<FMT, RND, NT>(u, v, ot, y, (uint32_t *)codes, scales, outer,
                                          seed_lo, seed_hi);
        } else {
            const uint4 v0 = x[2 * u], v1 = x[2 * u + 1];
            quant_row_seg<FMT, RND, NT>(u, v0, v1, ot, y, (uint2 *)codes, scales, outer,
                                        seed_lo, seed_hi);
        }
    }
}

// ---------------------------------------------------------------------------
// Column-axis kernels: lane = 8 columns x 16 rows
// ---------------------------------------------------------------------------
struct ColTile {
    uint32_t col0;   // first of the lane's 8 columns
    uint32_t row0;   // first of the lane's 16 rows
    uint32_t rb;     // lane's row block within its 8-lane group
    bool valid;
};

// One workgroup covers 64 columns x 512 rows (4 waves of 128 rows); the 1-D
// grid runs column tiles fastest.
__device__ __forceinline__ ColTile col_tile(uint32_t R, uint32_t C)
{
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t tiles_c = (C + 63) >> 6;
    ColTile t;
    t.rb = lane & 7;
    t.col0 = (blockIdx.x % tiles_c) * 64 + (lane >> 3) * 8;
    t.row0 = (((blockIdx.x / tiles_c) * 4 + wave) * 8 + t.rb) * 16;
    t.valid = t.col0 < C && t.row0 < R;
    return t;
}

__device__ __forceinline__ void seg_set_word(uint4 &v, int k, uint32_t w)
{
    if (k == 0) v.x = w;
    else if (k == 1) v.y = w;
    else if (k == 2) v.z = w;
    else v.w = w;
}
// Put the column-pair results of columns 2k and 2k+1 (pairs along rows) back
// into the row segments.
__device__ __forceinline__ void scatter_pairs(uint4 (&v)[16], int k, const uint32_t (&ya)[8],
                                              const uint32_t (&yb)[8])
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        seg_set_word(v[2 * i], k, (ya[i] & 0xFFFFu) | (yb[i] << 16));
        seg_set_word(v[2 * i + 1], k, (ya[i] >> 16) | (yb[i] & 0xFFFF0000u));
    }
}

// Quantizer tile: a lane holds 8 columns of 16 consecutive rows, eight lanes
// stack 128 rows, a wave spans 64 columns; the four waves of a workgroup sit
// kColWc side by side along the columns and 4 / kColWc along the rows.  The
// transposed codes, scales and outer scales are gathered in LDS and leave the
// workgroup as runs of kColTileR / 2, kColTileR / B and kColTileR / 128
// entries per column, instead of each lane storing its 8-byte and 1-byte
// pieces at column stride.
#ifndef FQ_COL_WC
#define FQ_COL_WC 4
#endif
constexpr uint32_t kColWc = FQ_COL_WC;
constexpr uint32_t kColTileC = 64 * kColWc, kColTileR = 128 * (4 / kColWc);
constexpr uint32_t kColCodePitch = kColTileR / 2 + 8;   // bytes; 8 * pitch = 64 mod 256

__device__ __forceinline__ uint32_t vword(const uint4 &v, int k)
{
    return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

struct QColTile {
    uint32_t col0, row0, rb;   // lane's first column, first row, row block in its group
    uint32_t lc, lr;           // the same relative to the workgroup tile
    uint32_t tc0, tr0;         // workgroup tile origin
    bool valid;
};

__device__ __forceinline__ QColTile quant_col_tile(uint32_t R, uint32_t C)
{
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t tiles_c = (C + kColTileC - 1) / kColTileC;
    QColTile t;
    t.rb = lane & 7;
    t.tc0 = (blockIdx.x % tiles_c) * kColTileC;
    t.tr0 = (blockIdx.x / tiles_c) * kColTileR;
    t.lc = (wave % kColWc) * 64 + (lane >> 3) * 8;
    t.lr = (wave / kColWc) * 128 + t.rb * 16;
    t.col0 = t.tc0 + t.lc;
    t.row0 = t.tr0 + t.lr;
    t.valid = t.col0 < C && t.row0 < R;
    return t;
}

template <int FMT, int RND, bool NT>
__global__ __launch_bounds__(kThreads) void k_quant_col(
    const uint4 *__restrict__ x, uint32_t R, uint32_t C, uint4 *__restrict__ y,
    uint4 *__restrict__ yt, uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
    float *__restrict__ outer, const uint32_t *__restrict__ partials, uint32_t npart,
    uint32_t seed_lo, uint32_t seed_hi)
{
    constexpr uint32_t B = (FMT == FMT_MX) ? 32 : 16;
    constexpr uint32_t SPB = kColTileR / B;          // scale bytes per column in the tile
    constexpr uint32_t OPB = kColTileR / 128;        // outer scales per column in the tile
    __shared__ __attribute__((aligned(16))) uint8_t s_codes[kColTileC * kColCodePitch];
    __shared__ uint8_t s_scales[kColTileC * SPB];
    __shared__ float s_outer[FMT == FMT_NV128 ? kColTileC * OPB : 1];

    OuterScale ot = {0.0f, 0.0f};
    if (FMT == FMT_NVT) {
        ot = tensor_scale(partials, npart);
        if (outer && blockIdx.x == 0 && threadIdx.x == 0) outer[0] = ot.s;
    }
    const QColTile t = quant_col_tile(R, C);
    const uint32_t ldx = C >> 3;   // 16-byte segments per row

    if (t.valid) {     // MXFP4 pairs and double-block groups are valid together
        uint4 v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = x[(size_t)(t.row0 + r) * ldx + (t.col0 >> 3)];

        // per-column maxima of the lane's 16 rows: packed u16 max
        uint32_t mw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int k = 0; k < 4; ++k) mw[k] = pkmax_u16(mw[k], vword(v[r], k) & 0x7FFF7FFFu);

#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t yph[2][8];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t c = 2 * k + h;
                const uint32_t col = t.col0 + c;
                const uint32_t amax16 = h ? (mw[k] >> 16) : (mw[k] & 0xFFFFu);
                float so = 0.0f;
                const BlockScale b = lane_block_scale<FMT>(amax16, ot, so);
                if (FMT == FMT_NV128 && t.rb == 0) s_outer[(t.lc + c) * OPB + t.lr / 128] = so;
                if (FMT != FMT_MX || (t.rb & 1) == 0)
                    s_scales[(t.lc + c) * SPB + t.lr / B] = (uint8_t)b.code;
                u32x4 rnd[2];
                if (RND == RND_SR) {
                    const uint64_t call0 = ((uint64_t)col * R + t.row0) >> 3;
                    rnd[0] = philox4x32_10((uint32_t)call0, (uint32_t)(call0 >> 32), 0u, 0u,
                                           seed_lo, seed_hi);
                    rnd[1] = philox4x32_10((uint32_t)(call0 + 1), (uint32_t)((call0 + 1) >> 32),
                                           0u, 0u, seed_lo, seed_hi);
                }
                // column pairs along rows: element 2i in the low half of xp[i]
                uint32_t xp[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t wa = vword(v[2 * i], k), wb = vword(v[2 * i + 1], k);
                    xp[i] = h ? ((wa >> 16) | (wb & 0xFFFF0000u)) : ((wa & 0xFFFFu) | (wb << 16));
                }
                uint32_t cw[2];
                encode_pairs<FMT, RND, 8>(xp, b, rnd, cw, yph[h]);
                *reinterpret_cast<uint2 *>(&s_codes[(t.lc + c) * kColCodePitch + t.lr / 2]) =
                    make_uint2(cw[0], cw[1]);
                if (yt) {
                    uint4 *dst = yt + (((size_t)col * R + t.row0) >> 3);
                    st_stream<NT>(&dst[0], make_uint4(yph[h][0], yph[h][1], yph[h][2], yph[h][3]));
                    st_stream<NT>(&dst[1], make_uint4(yph[h][4], yph[h][5], yph[h][6], yph[h][7]));
                }
            }
            if (y) {
                // columns 2k, 2k+1 back into the row segments
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    seg_set_word(v[2 * i], k, (yph[0][i] & 0xFFFFu) | (yph[1][i] << 16));
                    seg_set_word(v[2 * i + 1], k, (yph[0][i] >> 16) | (yph[1][i] & 0xFFFF0000u));
                }
            }
        }
        if (y) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                st_stream<NT>(&y[(size_t)(t.row0 + r) * ldx + (t.col0 >> 3)], v[r]);
        }
    }
    __syncthreads();

    // The tile's transposed outputs, column by column.  Only entries whose
    // column and rows exist are written (R is a multiple of B; a partial last
    // band of rows fills a prefix of each column's run).
    const uint32_t rows_here = min(kColTileR, R - t.tr0);
    if (codes) {
        constexpr uint32_t P8 = kColTileR / 16;      // 8-byte pieces per column
        for (uint32_t q = threadIdx.x; q < kColTileC * P8; q += kThreads) {
            const uint32_t lc = q / P8, j = q % P8;
            if (t.tc0 + lc < C && j * 16 < rows_here)
                st_stream<NT>(reinterpret_cast<uint2 *>(codes + (size_t)(t.tc0 + lc) * (R >> 1) +
                                                        (t.tr0 >> 1) + j * 8),
                              *reinterpret_cast<const uint2 *>(&s_codes[lc * kColCodePitch + j * 8]));
        }
    }
    if (scales) {
        for (uint32_t q = threadIdx.x; q < kColTileC * SPB; q += kThreads) {
            const uint32_t lc = q / SPB, j = q % SPB;
            if (t.tc0 + lc < C && j * B < rows_here)
                scales[(size_t)(t.tc0 + lc) * (R / B) + t.tr0 / B + j] = s_scales[q];
        }
    }
    if (FMT == FMT_NV128 && outer) {
        for (uint32_t q = threadIdx.x; q < kColTileC * OPB; q += kThreads) {
            const uint32_t lc = q / OPB, j = q % OPB;
            if (t.tc0 + lc < C && j * 128 < rows_here)
                outer[(size_t)(t.tc0 + lc) * (R >> 7) + (t.tr0 >> 7) + j] = s_outer[q];
        }
    }
}

// ---------------------------------------------------------------------------
// Dequantize
// ---------------------------------------------------------------------------
template <int FMT>
__device__ __forceinline__ float stored_s_eff(uint32_t code, float s)
{
    return (FMT == FMT_MX) ? e8m0_value(code) : e4m3_value(code) * s;
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_dequant_row(
    const uint32_t *__restrict__ codes, const uint8_t *__restrict__ scales,
    const float *__restrict__ outer, uint32_t nchunks, uint4 *__restrict__ y)
{
    const float s_t = (FMT == FMT_NVT) ? outer[0] : 0.0f;
    for (uint32_t c = blockIdx.x * kThreads + threadIdx.x; c < nchunks;
         c += gridDim.x * kThreads) {
        const uint32_t cw = codes[c];
        float s = s_t;
        if (FMT == FMT_NV128) s = outer[c >> 4];
        const float se = stored_s_eff<FMT>(scales[FMT == FMT_MX ? (c >> 2) : (c >> 1)], s);
        uint32_t yp[4];
        decode8<FMT>(cw, se, yp);
        st_stream<true>(&y[c], make_uint4(yp[0], yp[1], yp[2], yp[3]));
    }
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_dequant_col(
    const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
    const float *__restrict__ outer, uint32_t R, uint32_t C, uint4 *__restrict__ y)
{
    constexpr uint32_t B = (FMT == FMT_MX) ? 32 : 16;
    const ColTile t = col_tile(R, C);
    if (!t.valid) return;
    const uint32_t ldx = C >> 3;
    uint4 v[16];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t yph[2][8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t col = t.col0 + 2 * k + h;
            const uint2 cw =
                *reinterpret_cast<const uint2 *>(codes + (size_t)col * (R >> 1) + (t.row0 >> 1));
            float s = 0.0f;
            if (FMT == FMT_NVT) s = outer[0];
            if (FMT == FMT_NV128) s = outer[(size_t)col * (R >> 7) + (t.row0 >> 7)];
            const float se = stored_s_eff<FMT>(scales[(size_t)col * (R / B) + t.row0 / B], s);
            decode8<FMT>(cw.x, se, &yph[h][0]);
            decode8<FMT>(cw.y, se, &yph[h][4]);
        }
        scatter_pairs(v, k, yph[0], yph[1]);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) st_stream<true>(&y[(size_t)(t.row0 + r) * ldx + (t.col0 >> 3)], v[r]);
}

// ---------------------------------------------------------------------------
// Straight-through estimator with clipping mask
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ste_word(uint32_t dyw, uint32_t keep, int bit)
{
    return (((keep >> bit) & 1u) ? (dyw & 0xFFFFu) : 0u) |
           (((keep >> (bit + 1)) & 1u) ? (dyw & 0xFFFF0000u) : 0u);
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
        const BlockScale b = scale_from_code<FMT>(scales[FMT == FMT_MX ? (c >> 2) : (c >> 1)], s);
        const uint32_t xp[4] = {v.x, v.y, v.z, v.w};
        const uint32_t keep = keep_mask<FMT, 4>(xp, b);
        st_stream<true>(&dx[c], make_uint4(ste_word(d.x, keep, 0), ste_word(d.y, keep, 2),
                                           ste_word(d.z, keep, 4), ste_word(d.w, keep, 6)));
    }
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_ste_col(
    const uint4 *__restrict__ x, const uint8_t *__restrict__ scales,
    const float *__restrict__ outer, const uint4 *__restrict__ dy, uint32_t R, uint32_t C,
    uint4 *__restrict__ dx)
{
    constexpr uint32_t B = (FMT == FMT_MX) ? 32 : 16;
    const ColTile t = col_tile(R, C);
    if (!t.valid) return;
    const uint32_t ldx = C >> 3;
    BlockScale bs[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint32_t col = t.col0 + c;
        float s = 0.0f;
        if (FMT == FMT_NVT) s = outer[0];
        if (FMT == FMT_NV128) s = outer[(size_t)col * (R >> 7) + (t.row0 >> 7)];
        bs[c] = scale_from_code<FMT>(scales[(size_t)col * (R / B) + t.row0 / B], s);
    }
#pragma unroll 4
    for (int r = 0; r < 16; ++r) {
        const size_t idx = (size_t)(t.row0 + r) * ldx + (t.col0 >> 3);
        const uint4 v = x[idx];
        const uint4 d = dy[idx];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t keep = 0;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const uint32_t xb = (c & 1) ? hi_bits(w[c >> 1]) : lo_bits(w[c >> 1]);
            keep |= (scaled_mag<FMT>(xb, bs[c]) <= 6.0f ? 1u : 0u) << c;
        }
        st_stream<true>(&dx[idx], make_uint4(ste_word(d.x, keep, 0), ste_word(d.y, keep, 2),
                                             ste_word(d.z, keep, 4), ste_word(d.w, keep, 6)));
    }
}

// ---------------------------------------------------------------------------
// launch helpers
// ---------------------------------------------------------------------------
uint32_t row_grid(uint64_t nseg, uint32_t per_block)
{
    uint64_t g = (nseg + per_block - 1) / per_block;
    if (g > kRowGridCap) g = kRowGridCap;
    if (g == 0) g = 1;
    return (uint32_t)g;
}

// Column-axis grid: one workgroup per 64-column x 512-row tile.
dim3 col_grid(int64_t R, int64_t C)
{
    uint64_t gx = (uint64_t)((C + 63) / 64);
    uint64_t gy = (uint64_t)((R + 511) / 512);
    return dim3((uint32_t)(gx * gy), 1, 1);
}

// Column-axis quantizer grid: one workgroup per kColTileC x kColTileR tile.
dim3 quant_col_grid(int64_t R, int64_t C)
{
    uint64_t gx = (uint64_t)((C + kColTileC - 1) / kColTileC);
    uint64_t gy = (uint64_t)((R + kColTileR - 1) / kColTileR);
    return dim3((uint32_t)(gx * gy), 1, 1);
}

template <int FMT, int RND, bool NT>
hipError_t quant_dispatch_nt(const fqimpl::QuantArgs &a, uint32_t npart, hipStream_t st)
{
    const uint32_t slo = (uint32_t)a.seed, shi = (uint32_t)(a.seed >> 32);
    const uint32_t *parts = a.partials;
    if (!a.col) {
        constexpr int MAP = (RND == RND_SR) ? 0 : 1;
        const uint64_t nunits = (uint64_t)a.R * a.C / (MAP == 1 ? 8 : 16);
        hipLaunchKernelGGL((k_quant_row<FMT, RND, MAP, NT>), dim3(row_grid(nunits, kThreads)),
                           dim3(kThreads), 0, st, (const uint4 *)a.x, (uint32_t)nunits,
                           (uint4 *)a.y, a.codes, (uint8_t *)a.scales, a.outer, parts, npart,
                           slo, shi);
    } else {
        hipLaunchKernelGGL((k_quant_col<FMT, RND, NT>), quant_col_grid(a.R, a.C), dim3(kThreads), 0,
                           st, (const uint4 *)a.x, (uint32_t)a.R, (uint32_t)a.C, (uint4 *)a.y,
                           (uint4 *)a.yt, (uint8_t *)a.codes, (uint8_t *)a.scales, a.outer,
                           parts, npart, slo, shi);
    }
    return hipGetLastError();
}

template <int FMT, int RND>
hipError_t quant_dispatch(const fqimpl::QuantArgs &a, uint32_t npart, hipStream_t st)
{
    return a.cached_outputs ? quant_dispatch_nt<FMT, RND, false>(a, npart, st)
                            : quant_dispatch_nt<FMT, RND, true>(a, npart, st);
}

}  // namespace

namespace fqimpl {

hipError_t launch_absmax(const void *x, int64_t n_elems, uint32_t *partials,
                         uint32_t *npart_out, hipStream_t stream)
{
    const uint64_t nchunks = (uint64_t)n_elems / 8;
    uint64_t g = (nchunks + kAbsmaxThreads * 4 - 1) / (kAbsmaxThreads * 4);
    if (g > kAbsmaxGrid) g = kAbsmaxGrid;
    if (g == 0) g = 1;
    hipLaunchKernelGGL(k_absmax, dim3((uint32_t)g), dim3(kAbsmaxThreads), 0, stream,
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
        hipLaunchKernelGGL(k_dequant_row<FMT>, dim3(row_grid(nchunks, kThreads)), dim3(kThreads),
                           0, st, (const uint32_t *)codes, (const uint8_t *)scales, outer,
                           (uint32_t)nchunks, (uint4 *)y);
    } else {
        hipLaunchKernelGGL(k_dequant_col<FMT>, col_grid(R, C), dim3(kThreads), 0, st,
                           (const uint8_t *)codes, (const uint8_t *)scales, outer, (uint32_t)R,
                           (uint32_t)C, (uint4 *)y);
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
        hipLaunchKernelGGL(k_ste_row<FMT>, dim3(row_grid(nchunks, kThreads)), dim3(kThreads), 0,
                           st, (const uint4 *)x, (const uint8_t *)scales, outer,
                           (const uint4 *)dy, (uint32_t)nchunks, (uint4 *)dx);
    } else {
        hipLaunchKernelGGL(k_ste_col<FMT>, col_grid(R, C), dim3(kThreads), 0, st,
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
