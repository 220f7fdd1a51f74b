// fq_hadamard.hip -- random Hadamard transform of BF16 tensors on gfx950.
//
// "Resumo Tecnico: TetraJet-v2", sec. 2.C (OutControl): the products of the
// backward pass are computed on operands rotated by a random Hadamard
// transform, which spreads the energy of outlier channels before the FP4
// quantizer sees them.  Rotating both operands of a product along its
// contraction axis by the same orthogonal (H S / sqrt(n)) leaves the product
// unchanged in exact arithmetic.
//
// Definition (blocks of n = 16 or 128 consecutive elements along the axis):
//   s_j = -1 where bit (j mod 128) of Philox4x32-10(key = seed,
//         counter = (j / 128, 0, 0, 0)) is set, bit t of word w being bit
//         32w + t; j is the position along the transformed axis;
//   v   = s o x, widened to FP32 (exact);
//   radix-2 butterflies in FP32, half-widths h = 1, 2, ..., n/2, each pair
//   (i, i + h) of a 2h-group -> (a + b, a - b)  (Sylvester order);
//   y   = BF16_RNE(RN32(c_n * v)), c_n the FP32 value nearest to 1/sqrt(n).
//
// Row axis: a lane owns 16 consecutive elements of a row (two 16-byte loads);
// the first four butterfly stages stay in the lane, and for n = 128 the last
// three pair lanes 1, 2 and 4 apart (a 128-element block is 8 consecutive
// lanes).  Column axis: the column quantizer's 64-column x 256-row LDS tile;
// a lane rotates one 16-row segment of one column (the fused quantizers'
// rht_segment), crossing lanes 1, 2 and 4 apart for n = 128.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fq_device.hpp"
#include "fq_internal.h"

namespace {

using namespace fqdev;

constexpr int kThreads = 256;

typedef uint32_t u32v4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void st_out(uint4 *p, const uint4 &v, bool nt)
{
    if (nt) __builtin_nontemporal_store((u32v4){v.x, v.y, v.z, v.w}, reinterpret_cast<u32v4 *>(p));
    else *p = v;
}

template <int N>
__global__ __launch_bounds__(kThreads) void k_hadamard_row(const uint4 *__restrict__ x,
                                                           uint32_t nseg, uint32_t C,
                                                           uint4 *__restrict__ y, float c_n,
                                                           uint32_t seed_lo, uint32_t seed_hi,
                                                           int nt)
{
    for (uint32_t u = blockIdx.x * kThreads + threadIdx.x; u < nseg; u += gridDim.x * kThreads) {
        const uint4 a = x[2 * u], b = x[2 * u + 1];
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        // position along the row (C / 16 < 2^30, so 32-bit arithmetic)
        const uint64_t col0 = (uint64_t)(u % (C >> 4)) * 16;
        const uint32_t bits = sign_bits16(col0, seed_lo, seed_hi);
        float v[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[2 * i] = flip(as_f(lo_bits(w[i])), bits, 2 * i);
            v[2 * i + 1] = flip(as_f(hi_bits(w[i])), bits, 2 * i + 1);
        }
        fwht16(v);
        if (N == 128) fwht_lanes(v, (uint32_t)(col0 >> 4) & 7);
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = bf16_pair_rne(c_n * v[2 * i], c_n * v[2 * i + 1]);
        st_out(&y[2 * u], make_uint4(o[0], o[1], o[2], o[3]), nt);
        st_out(&y[2 * u + 1], make_uint4(o[4], o[5], o[6], o[7]), nt);
    }
}

// Column transform through LDS, with the column quantizer's tile and lane
// mapping: a workgroup of 8 waves copies a 64-column x 256-row tile into LDS
// with direct loads, every lane rotates one 16-row segment of one column
// (the 8 lanes of a column's 128-row block are consecutive, so the
// cross-lane butterflies of a 128-block stay inside an 8-lane group), writes
// it back, and the tile leaves as full 128-byte row pieces.
template <int N>
__global__ __launch_bounds__(kQcThreads) void k_hadamard_col(const uint4 *__restrict__ x,
                                                             uint32_t R, uint32_t C,
                                                             uint4 *__restrict__ y,
                                                             uint32_t seed_lo, uint32_t seed_hi,
                                                             int nt)
{
    __shared__ __attribute__((aligned(1024))) uint8_t s_tile[kQcRows / 8 * kQcBlockBytes];
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t tiles_c = (C + kQcCols - 1) / kQcCols;
    const uint32_t tc0 = (blockIdx.x % tiles_c) * kQcCols;
    const uint32_t tr0 = (blockIdx.x / tiles_c) * kQcRows;
    const uint32_t ldx = C >> 3;
    __builtin_amdgcn_s_setprio(1);      // memory phases ahead of the arithmetic
    // wave w fills blocks 4w .. 4w+3; rows and chunks outside the tensor
    // re-read its last row / chunk (the segments they would feed are unused)
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i) {
        const uint32_t blk = wave * 4 + i;
        const uint32_t row = min(tr0 + blk * 8 + (lane >> 3), R - 1);
        const uint32_t chunk = min((tc0 >> 3) + (((lane & 7) ^ (blk >> 1)) & 7), ldx - 1);
        __builtin_amdgcn_global_load_lds((const void *)(x + (size_t)row * ldx + chunk),
                                         (lds_void *)(s_tile + blk * kQcBlockBytes), 16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __builtin_amdgcn_s_setprio(0);

    const uint32_t rl0 = ((wave >> 2) * 8 + (lane & 7)) * 16;   // the lane's first tile row
    const uint32_t row0 = tr0 + rl0;
#pragma unroll 1
    for (uint32_t u = 0; u < 2; ++u) {
        const uint32_t lc = (lane >> 3) + 8 * (wave & 3) + 32 * u;
        // a 128-row block's 8 lanes are valid together (R % N == 0)
        if (tc0 + lc >= C || row0 >= R) continue;
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
        rht_segment<N>(xp, row0, seed_lo, seed_hi);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t r = rl0 + 2 * i;
            *reinterpret_cast<uint16_t *>(s_tile + qc_offset(r, lc >> 3) + byte_in_chunk) =
                (uint16_t)xp[i];
            *reinterpret_cast<uint16_t *>(s_tile + qc_offset(r + 1, lc >> 3) + byte_in_chunk) =
                (uint16_t)(xp[i] >> 16);
        }
    }
    __syncthreads();
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (uint32_t i = 0; i < kQcRows * 8 / kQcThreads; ++i) {
        const uint32_t q = i * kQcThreads + threadIdx.x;
        const uint32_t r = q >> 3, chunk = q & 7;
        if (tr0 + r < R && tc0 + chunk * 8 < C)
            st_out(&y[(size_t)(tr0 + r) * ldx + (tc0 >> 3) + chunk],
                   *reinterpret_cast<const uint4 *>(s_tile + qc_offset(r, chunk)), nt != 0);
    }
}

}  // namespace

namespace fqimpl {

hipError_t launch_hadamard(const void *x, int64_t R, int64_t C, int col, int n, uint64_t seed,
                           void *y, bool cached, hipStream_t st)
{
    const float c_n = n == 16 ? 0.25f : __builtin_bit_cast(float, 0x3DB504F3u);
    const uint32_t slo = (uint32_t)seed, shi = (uint32_t)(seed >> 32);
    const int nt = cached ? 0 : 1;
    if (!col) {
        const uint64_t nseg = (uint64_t)R * C / 16;
        uint64_t g = (nseg + kThreads - 1) / kThreads;
        if (g > (1u << 20)) g = 1u << 20;
        if (n == 16)
            hipLaunchKernelGGL(k_hadamard_row<16>, dim3((uint32_t)g), dim3(kThreads), 0, st,
                               (const uint4 *)x, (uint32_t)nseg, (uint32_t)C, (uint4 *)y, c_n, slo,
                               shi, nt);
        else
            hipLaunchKernelGGL(k_hadamard_row<128>, dim3((uint32_t)g), dim3(kThreads), 0, st,
                               (const uint4 *)x, (uint32_t)nseg, (uint32_t)C, (uint4 *)y, c_n, slo,
                               shi, nt);
    } else {
        const dim3 grid((uint32_t)(((C + kQcCols - 1) / kQcCols) * ((R + kQcRows - 1) / kQcRows)));
        if (n == 16)
            hipLaunchKernelGGL(k_hadamard_col<16>, grid, dim3(kQcThreads), 0, st,
                               (const uint4 *)x, (uint32_t)R, (uint32_t)C, (uint4 *)y, slo, shi, nt);
        else
            hipLaunchKernelGGL(k_hadamard_col<128>, grid, dim3(kQcThreads), 0, st,
                               (const uint4 *)x, (uint32_t)R, (uint32_t)C, (uint4 *)y, slo, shi, nt);
    }
    return hipGetLastError();
}

}  // namespace fqimpl
