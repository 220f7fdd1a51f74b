// fq_kernels.hip -- streaming FP4 quantize / dequantize / STE kernels, gfx950.
//
// All kernels are HBM-bound streams.  A lane works on 16 consecutive
// elements along the quantization axis at a time (one NVFP4 block, half an
// MXFP4 block), and the BF16 tensors move as 16-byte vector accesses
// coalesced across the wavefront:
//
//  * Row axis (groups along the contiguous dimension): the tensor is a flat
//    array of 16-element segments (32 bytes of BF16).  Lane i of a wave owns
//    segment base+i, so an MXFP4 block is a lane pair and a 128-element outer
//    block is 8 lanes; block maxima are combined with DPP, without LDS.
//  * Column axis (groups of consecutive rows of one column, i.e. the rows of
//    x^T).  The quantizer, the dequantizer and the STE stage a 64-column x
//    256-row tile in LDS, so that the BF16 tensor moves as whole 128-byte row
//    pieces, and give each lane one 16-row segment of a column, the row-axis
//    work unit; see k_quant_col.
//
// Numerics follow fq_device.hpp; the op definitions are those of fq.h.
#include "fq_device.hpp"
#include "fq_internal.h"

using namespace fqdev;

namespace {

// Row-axis streams, chosen by measurement on MI355X (16384 x 4096 BF16):
//  - round-to-nearest kernels and the STE map one 8-element chunk to a lane
//    (every load and store instruction is one contiguous 1 KB run), the
//    dequantizer two chunks 64 apart (more bytes in flight for its small
//    code and scale reads);
//  - stochastic-rounding kernels, which carry more ALU work per element
//    (Philox and the SR encoder), map a 16-element segment to a lane,
//    halving the per-lane block scale work;
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
// Streaming load of an input read exactly once: the non-temporal hint keeps
// it from displacing other data in L2 and the Infinity Cache.  On the
// 16384x4096 step it took 4-5 us off the chunk-mapped row quantizers and the
// STE, whose inputs would otherwise push out what the next kernel reads; the
// SR segment kernel and the column kernels' direct LDS loads measured equal
// or slower with it, so they keep plain loads.
template <bool NT>
__device__ __forceinline__ uint4 ld_stream(const uint4 *p)
{
    if (!NT) return *p;
    const u32v4 v = __builtin_nontemporal_load(reinterpret_cast<const u32v4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------------------
// Per-tensor maximum: partial maxima of |x| (as BF16 magnitude bits), one per
// workgroup.  Consumers reduce the partials themselves, so no zero-filled
// accumulator and no atomics are needed.
// ---------------------------------------------------------------------------
// One workgroup of kAbsmaxThreads per partial; at most kAbsmaxGrid partials,
// so that every quantizer workgroup reduces at most 1 KB of them.  A thread
// keeps kAbsmaxUnroll 16-byte loads in flight per pass, and the workgroups of
// a tensor are sized so that all of them make the same number of passes.
// One launch serves up to two tensors (the QAT linear's X and W): workgroups
// 0 .. j0.groups - 1 reduce the first, the rest the second.
constexpr int kAbsmaxThreads = 1024;
constexpr uint32_t kAbsmaxUnroll = 8;
constexpr uint32_t kAbsmaxGrid = 256;
static_assert(kAbsmaxGrid <= fqimpl::kAbsmaxPartials, "partials fit the workspace");

struct AbsmaxJob {
    const uint4 *x;
    uint32_t nchunks;         // 16-byte chunks of x
    uint32_t *partials;       // one word per workgroup
    uint32_t groups;          // workgroups of this tensor
    const uint8_t *retain;    // MASK: retained columns (bit c mod 8 of byte c / 8)
    uint32_t cpr;             // MASK: chunks per row
};

// MASK: the columns whose bit is set in retain take no part in the maximum
// (retained FP8 channels).
template <bool MASK>
__global__ __launch_bounds__(kAbsmaxThreads) void k_absmax(AbsmaxJob j0, AbsmaxJob j1)
{
    __shared__ uint32_t red[kAbsmaxThreads / 64];
    const bool second = blockIdx.x >= j0.groups;
    const AbsmaxJob j = second ? j1 : j0;
    const uint32_t wg = second ? blockIdx.x - j0.groups : blockIdx.x;
    constexpr uint32_t per = kAbsmaxThreads * kAbsmaxUnroll;
    uint32_t m = 0;
    for (uint32_t base = wg * per; base < j.nchunks; base += j.groups * per) {
        // indexes past the end re-read the last chunk (the maximum is
        // idempotent), so that no load sits behind a branch and all
        // kAbsmaxUnroll of them are in flight together
        uint4 v[kAbsmaxUnroll];
#pragma unroll
        for (uint32_t u = 0; u < kAbsmaxUnroll; ++u) {
            const uint32_t c = min(base + u * kAbsmaxThreads + threadIdx.x, j.nchunks - 1);
            v[u] = j.x[c];
            if (MASK) {
                const uint32_t r = j.retain[c % j.cpr];
                v[u].x &= ~retained_halves(r, 0);
                v[u].y &= ~retained_halves(r, 2);
                v[u].z &= ~retained_halves(r, 4);
                v[u].w &= ~retained_halves(r, 6);
            }
        }
#pragma unroll
        for (uint32_t u = 0; u < kAbsmaxUnroll; ++u) m = max(m, absmax_bits_8(v[u]));
    }
    m = block_reduce_max<kAbsmaxThreads>(m, red);
    if (threadIdx.x == 0) j.partials[wg] = m;
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
                                              float *__restrict__ outer,
                                              uint16_t *__restrict__ keep, uint32_t seed_lo,
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
    if (keep) keep[seg] = (uint16_t)keep_mask<FMT, 8>(xp, b);
    if (codes) st_stream<NT>(&codes[seg], make_uint2(cw[0], cw[1]));
    if (y) {
        st_stream<NT>(&y[2 * seg], make_uint4(yp[0], yp[1], yp[2], yp[3]));
        st_stream<NT>(&y[2 * seg + 1], make_uint4(yp[4], yp[5], yp[6], yp[7]));
    }
}

template <int FMT, int RND, bool NT>
__device__ __forceinline__ void quant_row_chunk(uint32_t c, const uint4 &v, const OuterScale &ot,
                                                uint4 *__restrict__ y,
                                                uint32_t *__restrict__ codes,
                                                uint8_t *__restrict__ scales,
                                                float *__restrict__ outer,
                                                uint8_t *__restrict__ keep, uint32_t seed_lo,
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
    if (keep) keep[c] = (uint8_t)keep_mask<FMT, 4>(xp, b);
    if (codes) st_stream<NT>(&codes[c], cw[0]);
    if (y) st_stream<NT>(&y[c], make_uint4(yp[0], yp[1], yp[2], yp[3]));
}

// MAP = 1: one 8-element chunk per lane (units = chunks); MAP = 2: two
// chunks per lane, 64 apart; MAP = 0: one 16-element segment per lane
// (units = segments).
template <int FMT, int RND, int MAP, bool NT, int RHT = 0>
__global__ __launch_bounds__(kThreads) void k_quant_row(
    const uint4 *__restrict__ x, uint32_t nunits, uint4 *__restrict__ y,
    void *__restrict__ codes, uint8_t *__restrict__ scales, float *__restrict__ outer,
    void *__restrict__ keep, const uint32_t *__restrict__ partials, uint32_t npart,
    uint32_t seed_lo, uint32_t seed_hi, uint32_t C, uint32_t rs_lo, uint32_t rs_hi)
{
    OuterScale ot = {0.0f, 0.0f};
    if (FMT == FMT_NVT) {
        ot = tensor_scale<kThreads>(partials, npart);
        if (outer && blockIdx.x == 0 && threadIdx.x == 0) outer[0] = ot.s;
    }
    // The per-tensor format reads x a second time right after the maximum
    // pass: its workgroups walk the tensor from the end, so the first ones
    // find the part of x the maximum pass read last still in the Infinity
    // Cache, before this pass's own traffic displaces it.
    const uint32_t wg = (FMT == FMT_NVT) ? gridDim.x - 1 - blockIdx.x : blockIdx.x;
    if (MAP == 2) {
        // two chunks per lane, 64 apart (a wave covers 2 KB per pass), both
        // loads issued before either chunk is encoded; a chunk past the end
        // re-reads the last one and is not encoded (blocks and 128-blocks
        // are whole groups of lanes, so a DPP group is valid or not as a whole)
        const uint32_t lane = threadIdx.x & 63;
        const uint32_t stride = gridDim.x * kThreads * 2;
        for (uint32_t u0 = (wg * kThreads + (threadIdx.x & ~63u)) * 2 + lane; u0 < nunits;
             u0 += stride) {
            const uint32_t u1 = u0 + 64;
            const uint4 v0 = ld_stream<NT>(&x[u0]);
            const uint4 v1 = ld_stream<NT>(&x[min(u1, nunits - 1)]);
            quant_row_chunk<FMT, RND, NT>(u0, v0, ot, y, (uint32_t *)codes, scales, outer,
                                          (uint8_t *)keep, seed_lo, seed_hi);
            if (u1 < nunits)
                quant_row_chunk<FMT, RND, NT>(u1, v1, ot, y, (uint32_t *)codes, scales, outer,
                                              (uint8_t *)keep, seed_lo, seed_hi);
        }
        return;
    }
    for (uint32_t u = wg * kThreads + threadIdx.x; u < nunits;
         u += gridDim.x * kThreads) {
        if (MAP == 1) {
            const uint4 v = ld_stream<NT>(&x[u]);
            quant_row_chunk<FMT, RND, NT>(u, v, ot, y, (uint32_t *)codes, scales, outer,
                                          (uint8_t *)keep, seed_lo, seed_hi);
        } else {
            uint4 v0 = x[2 * u], v1 = x[2 * u + 1];
            if (RHT) {
                // the rotated segment (position along the row: (16 u) mod C)
                uint32_t xp[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                const uint64_t j0 = ((uint64_t)u * 16) % C;
                rht_segment<RHT>(xp, j0, rs_lo, rs_hi);
                v0 = make_uint4(xp[0], xp[1], xp[2], xp[3]);
                v1 = make_uint4(xp[4], xp[5], xp[6], xp[7]);
            }
            quant_row_seg<FMT, RND, NT>(u, v0, v1, ot, y, (uint2 *)codes, scales, outer,
                                        (uint16_t *)keep, seed_lo, seed_hi);
        }
    }
}

// ---------------------------------------------------------------------------
// Column-axis kernels on a kQcCols x kQcRows tile staged in LDS
// ---------------------------------------------------------------------------
// Column quantizer: the tile goes through LDS, so that every lane works on
// one 16-row segment of one column at a time, exactly like a row-axis lane on
// its 16-element segment (same block scale, draws and encoder), with a small
// register footprint.
//
//  * A workgroup of 8 waves owns a kQcCols x kQcRows tile (64 columns x 256
//    rows).  Its waves copy it into LDS with direct loads
//    (global_load_lds_dwordx4: no registers, 1 KB of 8 full 128-byte row
//    pieces per instruction).  LDS block b holds tile rows 8b .. 8b+7, 128
//    bytes each; the 16-byte chunk of columns 8g .. 8g+7 of a row in block b
//    sits in slot g ^ ((b >> 1) & 7), so the eight segments a wave reads at
//    once (8 row blocks of one chunk) hit eight different slots, i.e. all
//    banks.
//  * Waves 0-3 take tile rows 0-127, waves 4-7 rows 128-255.  Lane l of wave
//    w takes row block rb = l & 7 (16 rows) of its half, in tile columns
//    (l >> 3) + 8 (w & 3) + 32 u, u = 0, 1.  The eight lanes of a column are
//    consecutive, so an MXFP4 block is a lane pair and the double block's
//    128-row outer block is the 8 lanes, as on the row axis.
//  * Codes, scales and outer scales are transposed outputs ([C, R/2],
//    [C, R/B], [C, R/128]): 256 rows of one column are one 128-byte line of
//    codes.  They are collected in LDS and leave after the tile is done as
//    whole lines (16 lanes of 8 bytes per column), 4-byte scale words and
//    8-byte outer pairs, instead of the 64-byte half lines one 128-row half
//    would give.  The fake-quantized BF16 values replace the inputs in LDS
//    and leave as full row pieces.
// (tile constants and qc_offset: fq_device.hpp)

// RET: retained FP8 channels (columns of x, bit mask retain [C/8], scales
// chan_scale [C]): every block of a retained column is empty for the FP4
// encoding (codes 0, scale of a zero block) and its values are the FP8 fake
// quantization under the channel's scale.
template <int FMT, int RND, bool NT, int RHT = 0, bool RET = false>
__global__ __launch_bounds__(kQcThreads) void k_quant_col(
    const uint4 *__restrict__ x, uint32_t R, uint32_t C, uint4 *__restrict__ y,
    uint4 *__restrict__ yt, uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
    float *__restrict__ outer, uint8_t *__restrict__ keep,
    const uint32_t *__restrict__ partials, uint32_t npart, uint32_t seed_lo, uint32_t seed_hi,
    uint32_t rs_lo, uint32_t rs_hi, const uint8_t *__restrict__ retain,
    const float *__restrict__ chan_scale)
{
    constexpr uint32_t B = (FMT == FMT_MX) ? 32 : 16;
    constexpr uint32_t NS = kQcRows / B;                  // scales per column of the tile
    __shared__ __attribute__((aligned(1024))) uint8_t s_tile[kQcRows / 8 * kQcBlockBytes];
    // the tile's codes (segment g of column c at 128 c + 8 g), scales (column
    // c, block k at NS c + k) and outer scales (column c, half h at 2 c + h)
    __shared__ __attribute__((aligned(16))) uint8_t s_codes[kQcCols * kQcSegs * 8];
    __shared__ __attribute__((aligned(16))) uint8_t s_scales[kQcCols * NS];
    __shared__ float s_outer[kQcCols * 2];
    // clip bits of the tile for the keep mask: row r, columns 32h .. 32h + 31
    // in word 2r + h (clipped elements are rare, so they are the ones set)
    __shared__ uint32_t s_clip[kQcRows * (kQcCols / 32)];
    static_assert(kQcRows * (kQcCols / 32) == kQcThreads, "one clip word per thread");

    OuterScale ot = {0.0f, 0.0f};
    if (FMT == FMT_NVT) {
        ot = tensor_scale<kQcThreads>(partials, npart);
        if (outer && blockIdx.x == 0 && threadIdx.x == 0) outer[0] = ot.s;
    }
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t tiles_c = (C + kQcCols - 1) / kQcCols;
    // per-tensor format: tiles in reverse order, as in k_quant_row (x was
    // just read by the maximum pass)
    const uint32_t tile = (FMT == FMT_NVT) ? gridDim.x - 1 - blockIdx.x : blockIdx.x;
    const uint32_t tc0 = (tile % tiles_c) * kQcCols;
    const uint32_t tr0 = (tile / tiles_c) * kQcRows;
    const uint32_t ldx = C >> 3;                     // 16-byte chunks per row
    // Waves issuing loads or stores run at a raised priority, so that on a CU
    // shared by several tiles the memory phases go ahead of the arithmetic
    // (about 1 us on 16384x4096)
    __builtin_amdgcn_s_setprio(1);

    // Direct loads: wave w fills blocks 4w .. 4w+3; lane l brings row l >> 3
    // of the block into slot l & 7, i.e. global chunk (l & 7) ^ (b >> 1).
    // Rows and chunks outside the tensor re-read its last row / chunk (the
    // segments they would feed are never used).
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i) {
        const uint32_t blk = wave * 4 + i;
        const uint32_t row = min(tr0 + blk * 8 + (lane >> 3), R - 1);
        const uint32_t chunk = min((tc0 >> 3) + (((lane & 7) ^ (blk >> 1)) & 7), ldx - 1);
        __builtin_amdgcn_global_load_lds((const void *)(x + (size_t)row * ldx + chunk),
                                         (lds_void *)(s_tile + blk * kQcBlockBytes), 16, 0, 0);
    }
    if (keep) s_clip[threadIdx.x] = 0u;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __builtin_amdgcn_s_setprio(0);

    const uint32_t rb = lane & 7, half = wave >> 2;
    const uint32_t seg = half * 8 + rb;              // this lane's segment of each column
    const uint32_t rl0 = seg * 16;                   // its first tile row
    const uint32_t row0 = tr0 + rl0;
#pragma unroll 1
    for (uint32_t u = 0; u < 2; ++u) {
        const uint32_t lc = (lane >> 3) + 8 * (wave & 3) + 32 * u;
        const uint32_t col = tc0 + lc;
        // MXFP4 pairs and double-block groups share their column and are
        // valid together (R is a multiple of B, and of 128 for the double block)
        if (col >= C || row0 >= R) continue;
        const uint32_t byte_in_chunk = (lc & 7) * 2;
        uint32_t xp[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t r = rl0 + 2 * i;
            const uint32_t lo = *reinterpret_cast<const uint16_t *>(
                s_tile + qc_offset(r, lc >> 3) + byte_in_chunk);
            const uint32_t hi = *reinterpret_cast<const uint16_t *>(
                s_tile + qc_offset(r + 1, lc >> 3) + byte_in_chunk);
            xp[i] = lo | (hi << 16);
        }
        // the rotation along the column (a 128-block is the lane's 8-lane group)
        if (RHT) rht_segment<RHT>(xp, row0, rs_lo, rs_hi);
        bool ret = false;
        uint32_t xr[8];
        BlockScale chs;
        if (RET) {
            ret = ((retain[col >> 3] >> (col & 7)) & 1u) != 0;
            chs.s_eff = ret ? chan_scale[col] : 0.0f;
            chs.code = 0;
            finish_nv_scale(chs);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                xr[i] = xp[i];
                if (ret) xp[i] = 0u;       // no part in any FP4 maximum, code 0
            }
        }
        float so = 0.0f;
        const BlockScale b = lane_block_scale<FMT>(absmax_bits_pairs8(xp), ot, so);
        if (FMT == FMT_NV128 && rb == 0) s_outer[lc * 2 + half] = so;
        if (FMT != FMT_MX) s_scales[lc * NS + seg] = (uint8_t)b.code;
        else if ((rb & 1) == 0) s_scales[lc * NS + seg / 2] = (uint8_t)b.code;
        u32x4 rnd[2];
        if (RND == RND_SR) {
            const uint64_t call0 = ((uint64_t)col * R + row0) >> 3;
            rnd[0] = philox4x32_10((uint32_t)call0, (uint32_t)(call0 >> 32), 0u, 0u, seed_lo,
                                   seed_hi);
            rnd[1] = philox4x32_10((uint32_t)(call0 + 1), (uint32_t)((call0 + 1) >> 32), 0u, 0u,
                                   seed_lo, seed_hi);
        }
        uint32_t cw[2], yq[8];
        encode_pairs<FMT, RND, 8>(xp, b, rnd, cw, yq);
        uint32_t clipped = keep ? ~keep_mask<FMT, 8>(xp, b) & 0xFFFFu : 0u;
        if (RET && ret) {
            clipped = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                bool c0, c1;
                yq[i] = fp8_fake_pair(xr[i], chs, chs, &c0, &c1);
                clipped |= (c0 ? 1u : 0u) << (2 * i) | (c1 ? 1u : 0u) << (2 * i + 1);
            }
        }
        if (keep) {
            // element i of the segment is row rl0 + i of the tile
            for (uint32_t clip = clipped; clip; clip &= clip - 1) {
                const uint32_t i = __builtin_ctz(clip);
                atomicOr(&s_clip[(rl0 + i) * (kQcCols / 32) + (lc >> 5)], 1u << (lc & 31));
            }
        }
        *reinterpret_cast<uint2 *>(s_codes + lc * (kQcSegs * 8) + seg * 8) = make_uint2(cw[0], cw[1]);
        if (yt) {
            uint4 *dst = yt + (((size_t)col * R + row0) >> 3);
            st_stream<NT>(&dst[0], make_uint4(yq[0], yq[1], yq[2], yq[3]));
            st_stream<NT>(&dst[1], make_uint4(yq[4], yq[5], yq[6], yq[7]));
        }
        if (y) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t r = rl0 + 2 * i;
                *reinterpret_cast<uint16_t *>(s_tile + qc_offset(r, lc >> 3) + byte_in_chunk) =
                    (uint16_t)yq[i];
                *reinterpret_cast<uint16_t *>(s_tile + qc_offset(r + 1, lc >> 3) + byte_in_chunk) =
                    (uint16_t)(yq[i] >> 16);
            }
        }
    }
    __syncthreads();
    __builtin_amdgcn_s_setprio(1);
    const uint32_t t = threadIdx.x;
    if (codes) {
        // 16 threads per column, 8 bytes (one segment) each: a wave stores four
        // whole 128-byte lines
#pragma unroll
        for (uint32_t p = 0; p < 2; ++p) {
            const uint32_t q = p * kQcThreads + t;
            const uint32_t c = q / kQcSegs, g = q % kQcSegs;
            if (tc0 + c < C && tr0 + g * 16 < R)
                st_stream<NT>(reinterpret_cast<uint2 *>(codes + (size_t)(tc0 + c) * (R >> 1) +
                                                        ((tr0 + g * 16) >> 1)),
                              *reinterpret_cast<const uint2 *>(s_codes + q * 8));
        }
    }
    if (scales && t < kQcCols * NS / 4) {
        // four consecutive scale bytes of one column per thread
        const uint32_t c = t / (NS / 4), k0 = (t % (NS / 4)) * 4;
        const uint32_t first_row = tr0 + k0 * B;
        if (tc0 + c < C && first_row < R) {
            const uint32_t w = *reinterpret_cast<const uint32_t *>(s_scales + t * 4);
            uint8_t *dst = scales + (size_t)(tc0 + c) * (R / B) + first_row / B;
            if (R % (4 * B) == 0) {
                *reinterpret_cast<uint32_t *>(dst) = w;
            } else {
                for (uint32_t k = 0; k < 4 && first_row + k * B < R; ++k)
                    dst[k] = (uint8_t)(w >> (8 * k));
            }
        }
    }
    if (FMT == FMT_NV128 && outer && t < kQcCols) {
        const uint32_t c = t;
        if (tc0 + c < C && tr0 < R) {
            float *dst = outer + (size_t)(tc0 + c) * (R >> 7) + (tr0 >> 7);
            if (R % 256 == 0) {
                *reinterpret_cast<float2 *>(dst) = make_float2(s_outer[2 * c], s_outer[2 * c + 1]);
            } else {
                dst[0] = s_outer[2 * c];
                if (tr0 + 128 < R) dst[1] = s_outer[2 * c + 1];
            }
        }
    }
    if (keep) {
        // thread t: tile row t / 2, columns 32 (t % 2) .. + 31 of the keep mask
        const uint32_t r = t / (kQcCols / 32), h = t % (kQcCols / 32);
        const uint32_t c0 = tc0 + 32 * h;
        if (tr0 + r < R && c0 < C) {
            const uint32_t kw = ~s_clip[t];
            uint8_t *dst = keep + ((size_t)(tr0 + r) * C + c0) / 8;
            if (c0 + 32 <= C && (((uintptr_t)dst) & 3) == 0) {
                *reinterpret_cast<uint32_t *>(dst) = kw;
            } else {
                const uint32_t nb = min(4u, (C - c0) / 8);
                for (uint32_t j = 0; j < nb; ++j) dst[j] = (uint8_t)(kw >> (8 * j));
            }
        }
    }
    if (!y) return;
    // the fake-quantized tile back to [R, C] as full 128-byte row pieces
#pragma unroll
    for (uint32_t i = 0; i < kQcRows * 8 / kQcThreads; ++i) {
        const uint32_t q = i * kQcThreads + t;
        const uint32_t r = q >> 3, chunk = q & 7;
        if (tr0 + r < R && tc0 + chunk * 8 < C)
            st_stream<NT>(&y[(size_t)(tr0 + r) * ldx + (tc0 >> 3) + chunk],
                          *reinterpret_cast<const uint4 *>(s_tile + qc_offset(r, chunk)));
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

constexpr uint32_t kDequantChunks = 2;

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_dequant_row(
    const uint32_t *__restrict__ codes, const uint8_t *__restrict__ scales,
    const float *__restrict__ outer, uint32_t nchunks, uint4 *__restrict__ y)
{
    // two chunks per lane, 64 apart, with all loads issued before any decode:
    // twice the bytes in flight per wave for the small code and scale reads
    constexpr uint32_t U = kDequantChunks;
    const float s_t = (FMT == FMT_NVT) ? outer[0] : 0.0f;
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t stride = gridDim.x * kThreads * U;
    for (uint32_t base = (blockIdx.x * kThreads + (threadIdx.x & ~63u)) * U; base < nchunks;
         base += stride) {
        uint32_t cw[U], sc[U];
        float s[U];
#pragma unroll
        for (uint32_t k = 0; k < U; ++k) {
            const uint32_t c = base + k * 64 + lane;
            const bool ok = c < nchunks;
            cw[k] = ok ? codes[c] : 0u;
            s[k] = s_t;
            if (FMT == FMT_NV128) s[k] = ok ? outer[c >> 4] : 0.0f;
            sc[k] = ok ? scales[FMT == FMT_MX ? (c >> 2) : (c >> 1)] : 0u;
        }
#pragma unroll
        for (uint32_t k = 0; k < U; ++k) {
            const uint32_t c = base + k * 64 + lane;
            if (c >= nchunks) continue;
            uint32_t yp[4];
            decode8<FMT>(cw[k], stored_s_eff<FMT>(sc[k], s[k]), yp);
            st_stream<true>(&y[c], make_uint4(yp[0], yp[1], yp[2], yp[3]));
        }
    }
}

// Column-axis dequantizer on the column quantizer's 64-column x 256-row tile:
// each lane decodes one 16-row segment of two adjacent columns (8 code bytes
// each; the 16 lanes of a column read its 128-byte line of codes), writes the
// BF16 pairs into the tile in LDS, and the tile leaves as full 128-byte row
// pieces instead of the 16-byte column pieces a register transpose would give.
template <int FMT>
__global__ __launch_bounds__(kQcThreads) void k_dequant_col(
    const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
    const float *__restrict__ outer, uint32_t R, uint32_t C, uint4 *__restrict__ y)
{
    constexpr uint32_t B = (FMT == FMT_MX) ? 32 : 16;
    __shared__ __attribute__((aligned(1024))) uint8_t s_tile[kQcRows / 8 * kQcBlockBytes];
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t tiles_c = (C + kQcCols - 1) / kQcCols;
    const uint32_t tc0 = (blockIdx.x % tiles_c) * kQcCols;
    const uint32_t tr0 = (blockIdx.x / tiles_c) * kQcRows;
    const uint32_t ldx = C >> 3;
    const float s_t = (FMT == FMT_NVT) ? outer[0] : 0.0f;
    const uint32_t rl0 = ((wave >> 2) * 8 + (lane & 7)) * 16;   // the lane's first tile row
    const uint32_t row0 = tr0 + rl0;
    const uint32_t lc = 2 * ((lane >> 3) + 8 * (wave & 3));     // the lane's column pair
    if (tc0 + lc < C && row0 < R) {
        uint32_t yq[2][8];
#pragma unroll
        for (uint32_t h = 0; h < 2; ++h) {
            const uint32_t col = tc0 + lc + h;
            const uint2 cw =
                *reinterpret_cast<const uint2 *>(codes + (size_t)col * (R >> 1) + (row0 >> 1));
            float s = s_t;
            if (FMT == FMT_NV128) s = outer[(size_t)col * (R >> 7) + (row0 >> 7)];
            const float se = stored_s_eff<FMT>(scales[(size_t)col * (R / B) + row0 / B], s);
            decode8<FMT>(cw.x, se, &yq[h][0]);
            decode8<FMT>(cw.y, se, &yq[h][4]);
        }
        const uint32_t byte_in_chunk = (lc & 7) * 2;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t r = rl0 + 2 * i;
            *reinterpret_cast<uint32_t *>(s_tile + qc_offset(r, lc >> 3) + byte_in_chunk) =
                (yq[0][i] & 0xFFFFu) | (yq[1][i] << 16);
            *reinterpret_cast<uint32_t *>(s_tile + qc_offset(r + 1, lc >> 3) + byte_in_chunk) =
                (yq[0][i] >> 16) | (yq[1][i] & 0xFFFF0000u);
        }
    }
    __syncthreads();
#pragma unroll
    for (uint32_t i = 0; i < kQcRows * 8 / kQcThreads; ++i) {
        const uint32_t q = i * kQcThreads + threadIdx.x;
        const uint32_t r = q >> 3, chunk = q & 7;
        if (tr0 + r < R && tc0 + chunk * 8 < C)
            st_stream<true>(&y[(size_t)(tr0 + r) * ldx + (tc0 >> 3) + chunk],
                            *reinterpret_cast<const uint4 *>(s_tile + qc_offset(r, chunk)));
    }
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
        const uint4 v = ld_stream<true>(&x[c]);
        const uint4 d = ld_stream<true>(&dy[c]);
        float s = s_t;
        if (FMT == FMT_NV128) s = outer[c >> 4];
        const BlockScale b = scale_from_code<FMT>(scales[FMT == FMT_MX ? (c >> 2) : (c >> 1)], s);
        const uint32_t xp[4] = {v.x, v.y, v.z, v.w};
        const uint32_t keep = keep_mask<FMT, 4>(xp, b);
        st_stream<true>(&dx[c], make_uint4(ste_word(d.x, keep, 0), ste_word(d.y, keep, 2),
                                           ste_word(d.z, keep, 4), ste_word(d.w, keep, 6)));
    }
}

// Column-axis STE on the column quantizer's tile and lane mapping: the x tile
// (64 columns x 256 rows) arrives in LDS by direct loads while every thread
// loads its four 16-byte row pieces of dy into registers; each lane then
// recomputes the clip test of one 16-row segment of one column from x and
// the stored block scale and marks the clipped elements (rare) in an LDS bit
// mask, and every thread stores its dy pieces as dx with those elements +0.
template <int FMT>
__global__ __launch_bounds__(kQcThreads) void k_ste_col(
    const uint4 *__restrict__ x, const uint8_t *__restrict__ scales,
    const float *__restrict__ outer, const uint4 *__restrict__ dy, uint32_t R, uint32_t C,
    uint4 *__restrict__ dx)
{
    constexpr uint32_t B = (FMT == FMT_MX) ? 32 : 16;
    constexpr uint32_t PIECES = kQcRows * 8 / kQcThreads;   // row pieces per thread
    __shared__ __attribute__((aligned(1024))) uint8_t s_x[kQcRows / 8 * kQcBlockBytes];
    // clip bits: row r, columns 32h .. 32h + 31 in word 2r + h
    __shared__ uint32_t s_clip[kQcRows * (kQcCols / 32)];
    static_assert(kQcRows * (kQcCols / 32) == kQcThreads, "one clip word per thread");
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6, t = threadIdx.x;
    const uint32_t tiles_c = (C + kQcCols - 1) / kQcCols;
    const uint32_t tc0 = (blockIdx.x % tiles_c) * kQcCols;
    const uint32_t tr0 = (blockIdx.x / tiles_c) * kQcRows;
    const uint32_t ldx = C >> 3;
    __builtin_amdgcn_s_setprio(1);      // memory phases ahead of the arithmetic
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i) {
        const uint32_t blk = wave * 4 + i;
        const uint32_t row = min(tr0 + blk * 8 + (lane >> 3), R - 1);
        const uint32_t chunk = min((tc0 >> 3) + (((lane & 7) ^ (blk >> 1)) & 7), ldx - 1);
        __builtin_amdgcn_global_load_lds((const void *)(x + (size_t)row * ldx + chunk),
                                         (lds_void *)(s_x + blk * kQcBlockBytes), 16, 0, 0);
    }
    // this thread's dy pieces: tile row q >> 3, chunk q & 7 for q = i * 512 + t
    uint4 d[PIECES];
#pragma unroll
    for (uint32_t i = 0; i < PIECES; ++i) {
        const uint32_t q = i * kQcThreads + t;
        const uint32_t r = min(tr0 + (q >> 3), R - 1);
        const uint32_t chunk = min((tc0 >> 3) + (q & 7), ldx - 1);
        d[i] = ld_stream<true>(&dy[(size_t)r * ldx + chunk]);
    }
    s_clip[t] = 0u;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __builtin_amdgcn_s_setprio(0);

    const uint32_t rl0 = ((wave >> 2) * 8 + (lane & 7)) * 16;   // the lane's first tile row
    const uint32_t row0 = tr0 + rl0;
#pragma unroll 1
    for (uint32_t u = 0; u < 2; ++u) {
        const uint32_t lc = (lane >> 3) + 8 * (wave & 3) + 32 * u;
        const uint32_t col = tc0 + lc;
        if (col >= C || row0 >= R) continue;
        const uint32_t byte_in_chunk = (lc & 7) * 2;
        uint32_t xp[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t r = rl0 + 2 * i;
            const uint32_t lo = *reinterpret_cast<const uint16_t *>(
                s_x + qc_offset(r, lc >> 3) + byte_in_chunk);
            const uint32_t hi = *reinterpret_cast<const uint16_t *>(
                s_x + qc_offset(r + 1, lc >> 3) + byte_in_chunk);
            xp[i] = lo | (hi << 16);
        }
        float s = 0.0f;
        if (FMT == FMT_NVT) s = outer[0];
        if (FMT == FMT_NV128) s = outer[(size_t)col * (R >> 7) + (row0 >> 7)];
        const BlockScale b = scale_from_code<FMT>(scales[(size_t)col * (R / B) + row0 / B], s);
        // element i of the segment is row rl0 + i of the tile
        for (uint32_t clip = ~keep_mask<FMT, 8>(xp, b) & 0xFFFFu; clip; clip &= clip - 1) {
            const uint32_t i = __builtin_ctz(clip);
            atomicOr(&s_clip[(rl0 + i) * (kQcCols / 32) + (lc >> 5)], 1u << (lc & 31));
        }
    }
    __syncthreads();
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (uint32_t i = 0; i < PIECES; ++i) {
        const uint32_t q = i * kQcThreads + t;
        const uint32_t r = q >> 3, chunk = q & 7;
        if (tr0 + r < R && tc0 + chunk * 8 < C) {
            // the chunk's 8 columns are bits 8 (chunk & 3) .. + 7 of word 2r + chunk / 4
            const uint32_t keep =
                ~(s_clip[r * (kQcCols / 32) + (chunk >> 2)] >> (8 * (chunk & 3))) & 0xFFu;
            st_stream<true>(&dx[(size_t)(tr0 + r) * ldx + (tc0 >> 3) + chunk],
                            make_uint4(ste_word(d[i].x, keep, 0), ste_word(d[i].y, keep, 2),
                                       ste_word(d[i].z, keep, 4), ste_word(d[i].w, keep, 6)));
        }
    }
}

// Clipped STE from a keep mask: chunk c (8 elements) of dy and byte c of the
// mask.  dy and dx may be the same buffer (each lane reads its chunk before
// writing it), so they are not restrict-qualified.
__global__ __launch_bounds__(kThreads) void k_ste_mask(const uint8_t *__restrict__ keep,
                                                       const uint4 *dy, uint32_t nchunks,
                                                       uint4 *dx)
{
    for (uint32_t c = blockIdx.x * kThreads + threadIdx.x; c < nchunks;
         c += gridDim.x * kThreads) {
        const uint4 d = ld_stream<true>(&dy[c]);
        const uint32_t k = keep[c];
        st_stream<true>(&dx[c], make_uint4(ste_word(d.x, k, 0), ste_word(d.y, k, 2),
                                           ste_word(d.z, k, 4), ste_word(d.w, k, 6)));
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

// Column-axis grid (quantizer, dequantizer, STE): one workgroup per
// kQcCols x kQcRows tile.
dim3 quant_col_grid(int64_t R, int64_t C)
{
    uint64_t gx = (uint64_t)((C + kQcCols - 1) / kQcCols);
    uint64_t gy = (uint64_t)((R + kQcRows - 1) / kQcRows);
    return dim3((uint32_t)(gx * gy), 1, 1);
}

template <int FMT, int RND, bool NT>
hipError_t quant_dispatch_nt(const fqimpl::QuantArgs &a, uint32_t npart, hipStream_t st)
{
    const uint32_t slo = (uint32_t)a.seed, shi = (uint32_t)(a.seed >> 32);
    const uint32_t *parts = a.partials;
    const uint32_t rlo = (uint32_t)a.rht_seed, rhi = (uint32_t)(a.rht_seed >> 32);
    if (!a.col) {
        // one 16-element segment per lane for SR and for rotated inputs (a
        // Hadamard block is one lane or an 8-lane group), else one chunk of 8
        const uint64_t nseg = (uint64_t)a.R * a.C / 16, nchunk = (uint64_t)a.R * a.C / 8;
        const dim3 gs(row_grid(nseg, kThreads)), gc(row_grid(nchunk, kThreads)), b(kThreads);
#define FQ_ROW_ARGS(n)                                                                      \
    (const uint4 *)a.x, (uint32_t)(n), (uint4 *)a.y, a.codes, (uint8_t *)a.scales, a.outer, \
        a.keep, parts, npart, slo, shi, (uint32_t)a.C, rlo, rhi
        if (a.rht_n == 16)
            hipLaunchKernelGGL((k_quant_row<FMT, RND, 0, NT, 16>), gs, b, 0, st, FQ_ROW_ARGS(nseg));
        else if (a.rht_n == 128)
            hipLaunchKernelGGL((k_quant_row<FMT, RND, 0, NT, 128>), gs, b, 0, st, FQ_ROW_ARGS(nseg));
        else if (RND == RND_SR)
            hipLaunchKernelGGL((k_quant_row<FMT, RND, 0, NT>), gs, b, 0, st, FQ_ROW_ARGS(nseg));
        else if (FMT == FMT_NVT)
            // the per-tensor format's workgroups each reduce the partial maxima
            // first: two chunks per lane halve their number (69.2 -> 67.6 us
            // on 16384x4096; the other formats measured equal either way)
            hipLaunchKernelGGL((k_quant_row<FMT, RND, 2, NT>), dim3(row_grid((nchunk + 1) / 2, kThreads)),
                               b, 0, st, FQ_ROW_ARGS(nchunk));
        else
            hipLaunchKernelGGL((k_quant_row<FMT, RND, 1, NT>), gc, b, 0, st, FQ_ROW_ARGS(nchunk));
#undef FQ_ROW_ARGS
    } else {
#define FQ_COL_ARGS                                                                          \
    (const uint4 *)a.x, (uint32_t)a.R, (uint32_t)a.C, (uint4 *)a.y, (uint4 *)a.yt,          \
        (uint8_t *)a.codes, (uint8_t *)a.scales, a.outer, (uint8_t *)a.keep, parts, npart, slo, \
        shi, rlo, rhi, (const uint8_t *)a.retain, a.chan_scale
        const dim3 g = quant_col_grid(a.R, a.C), b(kQcThreads);
        if (a.retain)
            hipLaunchKernelGGL((k_quant_col<FMT, RND, NT, 0, true>), g, b, 0, st, FQ_COL_ARGS);
        else if (a.rht_n == 16)
            hipLaunchKernelGGL((k_quant_col<FMT, RND, NT, 16>), g, b, 0, st, FQ_COL_ARGS);
        else if (a.rht_n == 128)
            hipLaunchKernelGGL((k_quant_col<FMT, RND, NT, 128>), g, b, 0, st, FQ_COL_ARGS);
        else
            hipLaunchKernelGGL((k_quant_col<FMT, RND, NT>), g, b, 0, st, FQ_COL_ARGS);
#undef FQ_COL_ARGS
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

namespace {
AbsmaxJob absmax_job(const void *x, int64_t n_elems, uint32_t *partials, const void *retain,
                     int64_t cols)
{
    AbsmaxJob j;
    j.x = (const uint4 *)x;
    j.nchunks = (uint32_t)((uint64_t)n_elems / 8);
    j.partials = partials;
    const uint64_t per = (uint64_t)kAbsmaxThreads * kAbsmaxUnroll;
    const uint64_t passes = (j.nchunks + kAbsmaxGrid * per - 1) / (kAbsmaxGrid * per);
    uint64_t g = passes ? (j.nchunks + passes * per - 1) / (passes * per) : 1;
    j.groups = (uint32_t)(g ? g : 1);
    j.retain = (const uint8_t *)retain;
    j.cpr = retain ? (uint32_t)(cols / 8) : 1u;
    return j;
}
}  // namespace

hipError_t launch_absmax(const void *x, int64_t n_elems, uint32_t *partials,
                         uint32_t *npart_out, hipStream_t stream, const void *retain,
                         int64_t cols)
{
    const AbsmaxJob j = absmax_job(x, n_elems, partials, retain, cols);
    AbsmaxJob none = j;
    none.groups = 0;
    if (retain)
        hipLaunchKernelGGL(k_absmax<true>, dim3(j.groups), dim3(kAbsmaxThreads), 0, stream, j,
                           none);
    else
        hipLaunchKernelGGL(k_absmax<false>, dim3(j.groups), dim3(kAbsmaxThreads), 0, stream, j,
                           none);
    *npart_out = j.groups;
    return hipGetLastError();
}

hipError_t launch_absmax_pair(const void *x0, int64_t n0, uint32_t *partials0, uint32_t *npart0,
                              const void *x1, int64_t n1, uint32_t *partials1, uint32_t *npart1,
                              hipStream_t stream)
{
    const AbsmaxJob j0 = absmax_job(x0, n0, partials0, nullptr, 0);
    const AbsmaxJob j1 = absmax_job(x1, n1, partials1, nullptr, 0);
    hipLaunchKernelGGL(k_absmax<false>, dim3(j0.groups + j1.groups), dim3(kAbsmaxThreads), 0,
                       stream, j0, j1);
    *npart0 = j0.groups;
    *npart1 = j1.groups;
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
        hipLaunchKernelGGL(k_dequant_row<FMT>,
                           dim3(row_grid((nchunks + kDequantChunks - 1) / kDequantChunks, kThreads)),
                           dim3(kThreads),
                           0, st, (const uint32_t *)codes, (const uint8_t *)scales, outer,
                           (uint32_t)nchunks, (uint4 *)y);
    } else {
        hipLaunchKernelGGL(k_dequant_col<FMT>, quant_col_grid(R, C), dim3(kQcThreads), 0, st,
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
        hipLaunchKernelGGL(k_ste_col<FMT>, quant_col_grid(R, C), dim3(kQcThreads), 0, st,
                           (const uint4 *)x, (const uint8_t *)scales, outer, (const uint4 *)dy,
                           (uint32_t)R, (uint32_t)C, (uint4 *)dx);
    }
    return hipGetLastError();
}

hipError_t launch_ste_mask(const void *keep, const void *dy, int64_t R, int64_t C, void *dx,
                           hipStream_t stream)
{
    const uint64_t nchunks = (uint64_t)R * C / 8;
    hipLaunchKernelGGL(k_ste_mask, dim3(row_grid(nchunks, kThreads)), dim3(kThreads), 0, stream,
                       (const uint8_t *)keep, (const uint4 *)dy, (uint32_t)nchunks, (uint4 *)dx);
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
