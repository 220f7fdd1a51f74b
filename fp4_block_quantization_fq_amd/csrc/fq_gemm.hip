// fq_gemm.hip -- BF16 x BF16 -> FP32-accumulated -> BF16 GEMM on CDNA4 MFMA.
//
// C[M, N] = A[M, K] * Bt[N, K]^T, both operands K-contiguous ("NT"), which
// is how the QAT linear hands over the fake-quantized activations X_hat and
// the transposed fake-quantized weight W_hat^T.  This is the one dense
// contraction of the method (QAT linear forward: weights and activations are
// both fake-quantized, then multiplied in the wider type -- gpt-oss QAT
// tutorial, "NVFP4: The Next Generation"; TetraJet-v2, sec. 2).
//
// Tiling: a 256 x 256 output tile per 512-thread workgroup (2 x 4 waves of
// 128 x 64, two waves per SIMD), K step 64.  Operand tiles go straight from global memory into LDS with gfx950's
// global_load_lds_dwordx4 (no staging registers), double-buffered, so the
// loads of step k+1 overlap the MFMAs of step k.  Each wave issues
// v_mfma_f32_32x32x16_bf16 on (BM/64) x (BN/64) accumulator tiles.
//
// LDS layout: one 128-byte row per tile row (64 BF16 of K), its eight 16-byte
// chunks XOR-swizzled by (row >> 1) & 7, so the 32 rows an MFMA fragment read
// touches spread over all 16 chunk positions of two consecutive rows.  The
// direct loads write 1 KB per wave instruction in lane order; each lane picks
// the global chunk that belongs in its LDS slot.
//
// Workgroups are renumbered so that each XCD (the hardware deals workgroups
// round-robin over 8 XCDs, each with its own L2) works on a contiguous run of
// tiles, grouped 8 tile-rows at a time so that B strips are reused in L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fq_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

#ifndef FQ_GEMM_PIPE
#define FQ_GEMM_PIPE 0         // 1: barrier before the last K slice, fragments prefetched
#endif
#ifndef FQ_GEMM_WN
#define FQ_GEMM_WN 4           // waves along N (2 waves along M)
#endif

constexpr int BK = 64;
constexpr int ROW_BYTES = BK * 2;      // 128 bytes of K per tile row
constexpr int kWavesM = 2, kWavesN = FQ_GEMM_WN;
constexpr int kThreads = 64 * kWavesM * kWavesN;
constexpr int kXcds = 8;

#ifndef FQ_GEMM_SWZ
#define FQ_GEMM_SWZ 2
#endif
#ifndef FQ_GEMM_BM
#define FQ_GEMM_BM 256
#endif
#ifndef FQ_GEMM_BN
#define FQ_GEMM_BN 256
#endif
#ifndef FQ_GEMM_SCHED
#define FQ_GEMM_SCHED 1
#endif

// Chunk position of 16-byte K chunk `chunk` in LDS row `row`: any 8 rows
// r..r+7 (r a multiple of 8) get 8 different positions and any 16 rows two
// different halves, so a fragment read of 32 consecutive rows is free of
// bank conflicts whether the LDS serves 8 or 16 lanes of 16 bytes per cycle.
__device__ __forceinline__ int swz(int row, int chunk)
{
#if FQ_GEMM_SWZ == 0
    return chunk ^ ((row >> 1) & 7);
#elif FQ_GEMM_SWZ == 1
    return chunk ^ (row & 7);
#else
    return chunk ^ (row & 7) ^ ((row >> 3) & 1);
#endif
}

// Issue the direct loads of one BM-row (or BN-row) operand tile at k0 into
// LDS.  Wave w, instruction i covers tile rows [w*ROWS/4 + 8i, +8): lane l
// fills LDS slot (l & 7) of row (l >> 3) with the global chunk swizzled there.
template <int ROWS>
__device__ __forceinline__ void load_tile(const uint16_t *__restrict__ g, int row0, int nrows,
                                          int K, int k0, uint8_t *lds_tile, int wave, int lane)
{
    constexpr int PER_WAVE = ROWS / (kWavesM * kWavesN);
#pragma unroll
    for (int i = 0; i < PER_WAVE / 8; ++i) {
        const int r = wave * PER_WAVE + i * 8 + (lane >> 3);
        const int c = swz(r, lane & 7);
        const int gr = min(row0 + r, nrows - 1);       // clamp: rows past the end feed
        const uint16_t *src = g + (size_t)gr * K + k0 + c * 8;   // discarded outputs
        uint8_t *dst = lds_tile + (wave * PER_WAVE + i * 8) * ROW_BYTES;
        __builtin_amdgcn_global_load_lds((const void *)src, (lds_void *)dst, 16, 0, 0);
    }
}

template <int BM, int BN>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_nt(const uint16_t *__restrict__ A,
                                                         const uint16_t *__restrict__ Bt,
                                                         uint16_t *__restrict__ C, int M, int N,
                                                         int K)
{
    constexpr int WTM = BM / kWavesM, WTN = BN / kWavesN;  // wave tile
    constexpr int TM = WTM / 32, TN = WTN / 32;             // 32x32 tiles per wave
    constexpr int A_BYTES = BM * ROW_BYTES, B_BYTES = BN * ROW_BYTES;
    constexpr int STAGE = A_BYTES + B_BYTES;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STAGE];

    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int ntiles = tiles_m * tiles_n;
    const int b = blockIdx.x;
    int logical = b;
    if (ntiles % kXcds == 0) logical = (b % kXcds) * (ntiles / kXcds) + b / kXcds;
    const int group = 8;
    const int tiles_per_group = group * tiles_n;
    const int g = logical / tiles_per_group;
    const int first_m = g * group;
    const int gm = min(tiles_m - first_m, group);
    const int in_g = logical % tiles_per_group;
    const int tm = first_m + in_g % gm;
    const int tn = in_g / gm;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave / kWavesN, wn = wave % kWavesN;
    const int row_a0 = tm * BM, row_b0 = tn * BN;

    floatx16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int nk = K / BK;
#if FQ_GEMM_PIPE
    // Fragment reads of one 16-wide K slice from an LDS stage.
    auto read_frags = [&](const uint8_t *stage, int ks, bf16x8 (&fa)[TM], bf16x8 (&fb)[TN]) {
        const int c = ks * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = wm * WTM + i * 32 + (lane & 31);
            fa[i] = *reinterpret_cast<const bf16x8 *>(stage + r * ROW_BYTES + swz(r, c) * 16);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int r = wn * WTN + j * 32 + (lane & 31);
            fb[j] = *reinterpret_cast<const bf16x8 *>(stage + A_BYTES + r * ROW_BYTES + swz(r, c) * 16);
        }
    };
    // prologue: stages 0 and 1 in flight, stage 0 waited for
    load_tile<BM>(A, row_a0, M, K, 0, lds, wave, lane);
    load_tile<BN>(Bt, row_b0, N, K, 0, lds + A_BYTES, wave, lane);
    __builtin_amdgcn_s_waitcnt(0);
    if (nk > 1) {
        load_tile<BM>(A, row_a0, M, K, BK, lds + STAGE, wave, lane);
        load_tile<BN>(Bt, row_b0, N, K, BK, lds + STAGE + A_BYTES, wave, lane);
    }
    __syncthreads();
    bf16x8 fa[TM], fb[TN], na[TM], nb[TN];
    read_frags(lds, 0, fa, fb);

    for (int kt = 0; kt < nk; ++kt) {
        uint8_t *cur = lds + (kt & 1) * STAGE;
        uint8_t *nxt = lds + ((kt + 1) & 1) * STAGE;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            if (ks < BK / 16 - 1) {
                read_frags(cur, ks + 1, na, nb);
            } else {
                // every wave holds its last fragments of `cur`; stage kt+1 has landed
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                if (kt + 2 < nk) {
                    load_tile<BM>(A, row_a0, M, K, (kt + 2) * BK, cur, wave, lane);
                    load_tile<BN>(Bt, row_b0, N, K, (kt + 2) * BK, cur + A_BYTES, wave, lane);
                }
                if (kt + 1 < nk) read_frags(nxt, 0, na, nb);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j],
                                                                        0, 0, 0);
#pragma unroll
            for (int i = 0; i < TM; ++i) fa[i] = na[i];
#pragma unroll
            for (int j = 0; j < TN; ++j) fb[j] = nb[j];
        }
    }
#else
    load_tile<BM>(A, row_a0, M, K, 0, lds, wave, lane);
    load_tile<BN>(Bt, row_b0, N, K, 0, lds + A_BYTES, wave, lane);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        uint8_t *cur = lds + (kt & 1) * STAGE;
        if (kt + 1 < nk) {
            uint8_t *nxt = lds + ((kt + 1) & 1) * STAGE;
            load_tile<BM>(A, row_a0, M, K, (kt + 1) * BK, nxt, wave, lane);
            load_tile<BN>(Bt, row_b0, N, K, (kt + 1) * BK, nxt + A_BYTES, wave, lane);
        }
        const uint8_t *sa = cur, *sb = cur + A_BYTES;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int c = ks * 2 + (lane >> 5);             // 16-byte chunk of K
            bf16x8 af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm * WTM + i * 32 + (lane & 31);
                af[i] = *reinterpret_cast<const bf16x8 *>(sa + r * ROW_BYTES + swz(r, c) * 16);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int r = wn * WTN + j * 32 + (lane & 31);
                bfr[j] = *reinterpret_cast<const bf16x8 *>(sb + r * ROW_BYTES + swz(r, c) * 16);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j],
                                                                        0, 0, 0);
#if FQ_GEMM_SCHED == 1
            // interleave: one fragment read between MFMAs
            for (int q = 0; q < TM + TN; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
            }
#endif
        }
        __builtin_amdgcn_s_waitcnt(0);      // this wave's loads of step kt+1 have landed
        __syncthreads();                    // all loads landed, all reads of `cur` done
    }

#endif

    // epilogue: accumulator element v of lane l sits at row (v/4)*8 + (l/32)*4 + v%4,
    // column l%32 of its 32 x 32 tile
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = tn * BN + wn * WTN + j * 32 + (lane & 31);
            if (col >= N) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = tm * BM + wm * WTM + i * 32 + (v >> 2) * 8 +
                                (lane >> 5) * 4 + (v & 3);
                if (row < M) {
                    __bf16 h = (__bf16)acc[i][j][v];
                    C[(size_t)row * N + col] = __builtin_bit_cast(uint16_t, h);
                }
            }
        }
}

}  // namespace

namespace fqimpl {

hipError_t launch_gemm_bf16_nt(const void *a, const void *bt, void *c, int64_t M, int64_t N,
                               int64_t K, hipStream_t stream)
{
    constexpr int BM = FQ_GEMM_BM, BN = FQ_GEMM_BN;
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    hipLaunchKernelGGL((k_gemm_nt<BM, BN>), dim3((uint32_t)tiles), dim3(kThreads), 0, stream,
                       (const uint16_t *)a, (const uint16_t *)bt, (uint16_t *)c, (int)M,
                       (int)N, (int)K);
    return hipGetLastError();
}

}  // namespace fqimpl
