// fq_gemm.hip -- BF16 x BF16 -> FP32-accumulated -> BF16 GEMM on CDNA4 MFMA.
//
// C[M, N] = A[M, K] * Bt[N, K]^T, both operands K-contiguous ("NT"), which
// is how the QAT linear hands over the fake-quantized activations X_hat and
// the transposed fake-quantized weight W_hat^T.  This is the one dense
// contraction of the method (QAT linear forward: weights and activations are
// both fake-quantized, then multiplied in the wider type -- gpt-oss QAT
// tutorial, "NVFP4: The Next Generation"; TetraJet-v2, sec. 2).
//
// Tiling: 128 x 128 output tile per 256-thread workgroup (2 x 2 waves of
// 64 x 64), K step 64 staged through double-buffered, padded LDS.  Each wave
// issues v_mfma_f32_32x32x16_bf16 on 2 x 2 accumulator tiles.  Workgroups are
// renumbered so that tiles sharing A rows run on the same XCD (the hardware
// deals workgroups round-robin over the 8 XCDs, each with its own L2).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fq_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_STRIDE = BK + 8;     // bf16 elements per LDS row (16-byte pad)
constexpr int kThreads = 256;
constexpr int kXcds = 8;

__global__ __launch_bounds__(kThreads) void k_gemm_nt(const uint16_t *__restrict__ A,
                                                      const uint16_t *__restrict__ Bt,
                                                      uint16_t *__restrict__ C, int M, int N,
                                                      int K)
{
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * LDS_STRIDE];

    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int ntiles = tiles_m * tiles_n;
    // XCD-aware renumbering: hardware id b runs on XCD b % 8; give each XCD a
    // contiguous range of logical tiles.
    int b = blockIdx.x;
    int logical = b;
    if (ntiles % kXcds == 0) logical = (b % kXcds) * (ntiles / kXcds) + b / kXcds;
    // grouped order: 8 tile-rows share a B column strip
    const int group = 8;
    const int tiles_per_group = group * tiles_n;
    const int g = logical / tiles_per_group;
    const int first_m = g * group;
    const int gm = min(tiles_m - first_m, group);
    const int in_g = logical % tiles_per_group;
    const int tm = first_m + in_g % gm;
    const int tn = in_g / gm;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;

    // global -> LDS mapping: 8 threads per 64-element row, 32 rows per pass
    const int lr = tid >> 3, lk = (tid & 7) * 8;
    const int row_a0 = tm * BM, row_b0 = tn * BN;

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    uint4 ra[4], rb[4];
    auto gload = [&](int k0) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int r = lr + 32 * p;
            const int ga = row_a0 + r, gb = row_b0 + r;
            ra[p] = ga < M ? *reinterpret_cast<const uint4 *>(A + (size_t)ga * K + k0 + lk)
                           : make_uint4(0, 0, 0, 0);
            rb[p] = gb < N ? *reinterpret_cast<const uint4 *>(Bt + (size_t)gb * K + k0 + lk)
                           : make_uint4(0, 0, 0, 0);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int r = lr + 32 * p;
            *reinterpret_cast<uint4 *>(&sA[buf][r * LDS_STRIDE + lk]) = ra[p];
            *reinterpret_cast<uint4 *>(&sB[buf][r * LDS_STRIDE + lk]) = rb[p];
        }
    };

    const int nk = K / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int kk = ks * 16 + (lane >> 5) * 8;
            bf16x8 af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = wm * 64 + i * 32 + (lane & 31);
                af[i] = *reinterpret_cast<const bf16x8 *>(&sA[buf][r * LDS_STRIDE + kk]);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int c = wn * 64 + j * 32 + (lane & 31);
                bfr[j] = *reinterpret_cast<const bf16x8 *>(&sB[buf][c * LDS_STRIDE + kk]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j],
                                                                        0, 0, 0);
        }
        if (kt + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }

    // epilogue: accumulator element v of lane l sits at row (v/4)*8 + (l/32)*4 + v%4,
    // column l%32 of the 32 x 32 tile
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = tn * BN + wn * 64 + j * 32 + (lane & 31);
            if (col >= N) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = tm * BM + wm * 64 + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
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
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    hipLaunchKernelGGL(k_gemm_nt, dim3((uint32_t)tiles), dim3(kThreads), 0, stream,
                       (const uint16_t *)a, (const uint16_t *)bt, (uint16_t *)c, (int)M,
                       (int)N, (int)K);
    return hipGetLastError();
}

}  // namespace fqimpl
