// fq_gemm.hip -- BF16 x BF16 -> FP32-accumulated -> BF16 GEMM on CDNA4 MFMA.
//
// C[M, N] = A[M, K] * Bt[N, K]^T, both operands K-contiguous ("NT").  This is
// the one dense contraction of the method: the QAT linear multiplies the
// fake-quantized activations by the fake-quantized weight (gpt-oss QAT
// tutorial, "NVFP4: The Next Generation"; TetraJet-v2, sec. 2), and its
// backward multiplies the re-quantized gradient operands (TetraJet-v2,
// sec. 2.A).  Every operand is handed over K-contiguous: X_hat [M, K] and
// W_hat^T [N, K] in the forward; Q(dY) [M, N] and Q(W_hat) [K, N] for dX;
// Q(X_hat)^T [K, M] and Q(dY)^T [N, M] for dW.
//
// Tiling: a 256 x 256 output tile per 512-thread workgroup (2 x 4 waves of
// 128 x 64, two waves per SIMD), K step 64.  Operand tiles go straight from
// global memory into LDS with gfx950's global_load_lds_dwordx4 (no staging
// registers), double-buffered, so the loads of step k+1 overlap the MFMAs of
// step k.  Each wave issues v_mfma_f32_32x32x16_bf16 on 4 x 2 accumulator
// tiles, its fragment reads interleaved with the MFMAs.
//
// LDS layout: one 128-byte row per tile row (64 BF16 of K).  Its eight
// 16-byte chunks are XOR-swizzled by (row & 7) ^ ((row >> 3) & 1), so the
// 32 rows of a fragment read hit all chunk positions (no bank conflicts,
// measured).  The direct loads write 1 KB per wave instruction in lane
// order; each lane fetches the global chunk that belongs in its LDS slot.
//
// Epilogue: each wave writes its 128 x 64 BF16 tile into its own 16 KB of the
// idle stage buffers and stores it back as whole 128-byte row pieces (the
// accumulator layout alone gives 64-byte runs of 2-byte stores).
//
// Workgroups are renumbered so that each XCD (the hardware deals workgroups
// round-robin over 8 XCDs, each with its own L2) works on a contiguous run of
// tiles, grouped 8 tile-rows at a time so that B strips are reused in L2.
//
// One launch may carry two independent problems (the two products of the
// backward): their tiles share the grid, the longer one first, so the chip
// stays busy where either alone would leave a partial last wave.
//
// MXFP4 operands need no dequantization at all: gfx950's
// v_mfma_scale_f32_32x32x64_f8f6f4 multiplies E2M1 codes directly and applies
// one E8M0 scale per 32-element block of each operand row, which is exactly
// the MXFP4 encoding (OCP Microscaling v1.0).  k_gemm_mxfp4_nt streams the
// packed codes (16 bytes = one 32-element block = one fragment half) through
// the same LDS tiles and swizzle as the BF16 kernel, 256 K-elements per stage
// instead of 64, and stages each row's eight E8M0 scales of a stage in LDS.
// The products of codes times powers of two are exact, so the result equals
// the FP32-accumulated product of the dequantized operands.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fq_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int ROW_BYTES = BK * 2;      // 128 bytes of K per tile row
constexpr int kWavesM = 2, kWavesN = 4;
constexpr int kThreads = 64 * kWavesM * kWavesN;
constexpr int kXcds = 8;

struct Problem {
    const uint16_t *A;
    const uint16_t *Bt;
    uint16_t *C;
    const uint8_t *keep;   // STE keep mask of C (bit n mod 8 of byte n / 8), or null
    int M, N, K;
    int tiles;     // workgroups of this problem in the grid
};

__device__ __forceinline__ int swz(int row, int chunk)
{
    return chunk ^ (row & 7) ^ ((row >> 3) & 1);
}

// Epilogue of one wave's WTM x 64 output tile.  The accumulators go to the
// wave's own 16 KB of the (now idle) stage buffers as BF16 rows of 128 bytes
// (16-byte chunk g of row r in slot g ^ (r & 7), so the two row groups of a
// store instruction hit different banks), then leave as whole 128-byte row
// pieces: lane l stores chunk l & 7 of row 8k + (l >> 3).  A 16-byte chunk
// is 8 columns starting at a multiple of 8 and N is a multiple of 8, so it is
// valid or invalid as a whole and its keep bits are one byte.  Accumulator
// element v of lane l sits at row (v/4)*8 + (l/32)*4 + v%4, column l%32 of
// its 32 x 32 tile.
template <int TM, int TN>
__device__ __forceinline__ void store_wave_tile(const floatx16 (&acc)[TM][TN], uint8_t *ep,
                                                uint16_t *__restrict__ C,
                                                const uint8_t *__restrict__ keep, int row0,
                                                int col0, int M, int N, int lane)
{
    static_assert(TN * 32 * 2 == 128, "one 128-byte LDS row per tile row");
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
                const int c = j * 32 + (lane & 31);
                *reinterpret_cast<uint16_t *>(ep + r * 128 + (((c >> 3) ^ (r & 7)) << 4) +
                                              (c & 7) * 2) =
                    __builtin_bit_cast(uint16_t, (__bf16)acc[i][j][v]);
            }
    // the keep bytes of all chunks first, so that their loads overlap
    constexpr int NCH = TM * 32 / 8;
    uint32_t kb[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int row = row0 + k * 8 + (lane >> 3), col = col0 + (lane & 7) * 8;
        kb[k] = (keep && row < M && col < N) ? keep[((size_t)row * N + col) >> 3] : 0xFFu;
    }
    // the wave reads back only what it wrote itself: LDS executes one wave's
    // instructions in order, so no barrier is needed
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int r = k * 8 + (lane >> 3), g = lane & 7;
        const int row = row0 + r, col = col0 + g * 8;
        uint4 w = *reinterpret_cast<const uint4 *>(ep + r * 128 + ((g ^ (r & 7)) << 4));
        if (row < M && col < N) {
            const size_t n = (size_t)row * N + col;
            if (keep) {
                // zero the elements whose keep bit is clear
                const uint32_t b = kb[k];
                const uint32_t m0 = ((b & 1u) ? 0xFFFFu : 0u) | ((b & 2u) ? 0xFFFF0000u : 0u);
                const uint32_t m1 = ((b & 4u) ? 0xFFFFu : 0u) | ((b & 8u) ? 0xFFFF0000u : 0u);
                const uint32_t m2 = ((b & 16u) ? 0xFFFFu : 0u) | ((b & 32u) ? 0xFFFF0000u : 0u);
                const uint32_t m3 = ((b & 64u) ? 0xFFFFu : 0u) | ((b & 128u) ? 0xFFFF0000u : 0u);
                w = make_uint4(w.x & m0, w.y & m1, w.z & m2, w.w & m3);
            }
            *reinterpret_cast<uint4 *>(C + n) = w;
        }
    }
}

// Issue the direct loads of one ROWS-row operand tile at k0 into LDS.  Wave
// w, instruction i covers tile rows [w*ROWS/8 + 8i, +8): lane l fills LDS
// slot (l & 7) of row (l >> 3) with the global chunk swizzled there.  Rows
// past the end of the operand are clamped to its last row (their outputs are
// never stored).
template <int ROWS>
__device__ __forceinline__ void load_tile(const uint16_t *__restrict__ g, int row0, int nrows,
                                          int K, int k0, uint8_t *lds_tile, int wave, int lane)
{
    constexpr int PER_WAVE = ROWS / (kWavesM * kWavesN);
#pragma unroll
    for (int i = 0; i < PER_WAVE / 8; ++i) {
        const int r = wave * PER_WAVE + i * 8 + (lane >> 3);
        const int c = swz(r, lane & 7);
        const int gr = min(row0 + r, nrows - 1);
        const uint16_t *src = g + (size_t)gr * K + k0 + c * 8;
        uint8_t *dst = lds_tile + (wave * PER_WAVE + i * 8) * ROW_BYTES;
        __builtin_amdgcn_global_load_lds((const void *)src, (lds_void *)dst, 16, 0, 0);
    }
}

__global__ __launch_bounds__(kThreads, 1) void k_gemm_nt(Problem p0, Problem p1)
{
    constexpr int WTM = BM / kWavesM, WTN = BN / kWavesN;  // wave tile
    constexpr int TM = WTM / 32, TN = WTN / 32;             // 32x32 tiles per wave
    constexpr int A_BYTES = BM * ROW_BYTES, B_BYTES = BN * ROW_BYTES;
    constexpr int STAGE = A_BYTES + B_BYTES;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STAGE];

    // this workgroup's problem (uniform across the workgroup)
    const bool second = (int)blockIdx.x >= p0.tiles;
    const uint16_t *__restrict__ A = second ? p1.A : p0.A;
    const uint16_t *__restrict__ Bt = second ? p1.Bt : p0.Bt;
    uint16_t *__restrict__ C = second ? p1.C : p0.C;
    const uint8_t *__restrict__ keep = second ? p1.keep : p0.keep;
    const int M = second ? p1.M : p0.M, N = second ? p1.N : p0.N, K = second ? p1.K : p0.K;
    const int b = second ? (int)blockIdx.x - p0.tiles : (int)blockIdx.x;

    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int ntiles = tiles_m * tiles_n;
    if (b >= ntiles) return;           // padding workgroups (XCD alignment of the second problem)
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
            // the compiler's single-wave MFMA interleaving strategy: spreads the
            // fragment reads among the MFMAs (measured 2 % faster than one read
            // between MFMA pairs placed by hand)
            __builtin_amdgcn_iglp_opt(1);
        }
        __builtin_amdgcn_s_waitcnt(0);      // this wave's loads of step kt+1 have landed
        __syncthreads();                    // all loads landed, all reads of `cur` done
    }

    // epilogue through this wave's 16 KB of the stage buffers (all reads of
    // them ended at the last barrier)
    store_wave_tile<TM, TN>(acc, lds + wave * (WTM * WTN * 2), C, keep, tm * BM + wm * WTM,
                            tn * BN + wn * WTN, M, N, lane);
}

// ---------------------------------------------------------------------------
// MXFP4 x MXFP4 on the scaled FP4 matrix cores
// ---------------------------------------------------------------------------
typedef int v8i __attribute__((ext_vector_type(8)));

struct Fp4Problem {
    const uint8_t *A;    // E2M1 codes [M, K/2], element 2i in the low nibble of byte i
    const uint8_t *As;   // E8M0 scales [M, K/32]
    const uint8_t *B;    // codes [N, K/2]
    const uint8_t *Bs;   // scales [N, K/32]
    uint16_t *C;         // BF16 [M, N]
    const uint8_t *keep; // STE keep mask of C, or null
    int M, N, K;
    int tiles;
};

constexpr int FK = 256;            // K elements per stage: 128 bytes of codes per row
constexpr int FSB = FK / 32;       // E8M0 scales per row per stage

// Direct loads of one ROWS-row code tile (128 bytes per row) into LDS, as
// load_tile; chunks past the end of K load chunk 0 instead (never used).
template <int ROWS>
__device__ __forceinline__ void load_codes(const uint8_t *__restrict__ g, int row0, int nrows,
                                           size_t pitch, size_t off0, int valid_chunks,
                                           uint8_t *lds_tile, int wave, int lane)
{
    constexpr int PER_WAVE = ROWS / (kWavesM * kWavesN);
#pragma unroll
    for (int i = 0; i < PER_WAVE / 8; ++i) {
        const int r = wave * PER_WAVE + i * 8 + (lane >> 3);
        int c = swz(r, lane & 7);
        if (c >= valid_chunks) c = 0;
        const int gr = min(row0 + r, nrows - 1);
        const uint8_t *src = g + (size_t)gr * pitch + off0 + c * 16;
        uint8_t *dst = lds_tile + (wave * PER_WAVE + i * 8) * ROW_BYTES;
        __builtin_amdgcn_global_load_lds((const void *)src, (lds_void *)dst, 16, 0, 0);
    }
}

__global__ __launch_bounds__(kThreads, 1) void k_gemm_mxfp4_nt(Fp4Problem p0, Fp4Problem p1)
{
    constexpr int WTM = BM / kWavesM, WTN = BN / kWavesN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int A_BYTES = BM * ROW_BYTES, B_BYTES = BN * ROW_BYTES;
    constexpr int STAGE = A_BYTES + B_BYTES;
    // The two stage buffers are separate variables, and the loop below is
    // unrolled by two so that every access names its buffer statically: the
    // compiler then knows that the reads of one buffer cannot see the direct
    // loads in flight into the other, and inserts no wait for those loads
    // before the stage's fragment reads (one shared array indexed by kt & 1
    // makes it wait for them, serializing load and compute).
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[STAGE];
    // per stage and operand row (A rows, then B rows): its eight E8M0 scales,
    // block b of the stage in byte b
    __shared__ uint64_t sc0[BM + BN], sc1[BM + BN];

    const bool second = (int)blockIdx.x >= p0.tiles;
    const uint8_t *__restrict__ A = second ? p1.A : p0.A;
    const uint8_t *__restrict__ As = second ? p1.As : p0.As;
    const uint8_t *__restrict__ Bc = second ? p1.B : p0.B;
    const uint8_t *__restrict__ Bs = second ? p1.Bs : p0.Bs;
    uint16_t *__restrict__ C = second ? p1.C : p0.C;
    const uint8_t *__restrict__ keep = second ? p1.keep : p0.keep;
    const int M = second ? p1.M : p0.M, N = second ? p1.N : p0.N, K = second ? p1.K : p0.K;
    const int b = second ? (int)blockIdx.x - p0.tiles : (int)blockIdx.x;

    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int ntiles = tiles_m * tiles_n;
    if (b >= ntiles) return;
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
    const size_t pitch = (size_t)K / 2;
    const int nblk = K / 32, nsub = K / 64;          // scale blocks, 64-element MFMA steps
    const int nk = (K + FK - 1) / FK;
    // This thread stages the scales of one operand row (A rows first, then B
    // rows; rows past the end are clamped like the codes).  The row holds
    // nblk = K/32 bytes, an even number, so its 2-byte loads are aligned.
    const bool sc_b = tid >= BM;
    const uint8_t *sc_src = sc_b ? Bs + (size_t)min(row_b0 + tid - BM, N - 1) * nblk
                                 : As + (size_t)min(row_a0 + tid, M - 1) * nblk;

    floatx16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    auto issue_stage = [&](int kt, uint8_t *st) {
        const int valid_chunks = min(8, (K - kt * FK) / 32);
        load_codes<BM>(A, row_a0, M, pitch, (size_t)kt * (FK / 2), valid_chunks, st, wave, lane);
        load_codes<BN>(Bc, row_b0, N, pitch, (size_t)kt * (FK / 2), valid_chunks, st + A_BYTES,
                       wave, lane);
    };
    // The eight scales of stage kt as four 2-byte loads, issued without a
    // branch and consumed only at the end of the stage (so that no wait for
    // them lands before the MFMAs).  Past the end of K they re-read the row's
    // last two scales, which no product uses.
    auto load_scales = [&](int kt, uint32_t (&h)[FSB / 2]) {
#pragma unroll
        for (int q = 0; q < FSB / 2; ++q)
            h[q] = *reinterpret_cast<const uint16_t *>(sc_src + min(kt * FSB + 2 * q, nblk - 2));
    };
    auto pack_scales = [](const uint32_t (&h)[FSB / 2]) {
        return (uint64_t)(h[0] | (h[1] << 16)) | ((uint64_t)(h[2] | (h[3] << 16)) << 32);
    };

    // One stage: issue the loads of stage kt+1 into `nxt`, run the MFMAs of
    // stage kt from `cur`, then publish the next scales and wait for all.
    auto stage = [&](int kt, const uint8_t *cur, uint8_t *nxt, const uint64_t *scur,
                     uint64_t *snxt) {
        uint32_t h[FSB / 2];
        load_scales(kt + 1, h);
        if (kt + 1 < nk) issue_stage(kt + 1, nxt);
        // this lane's scale words for the stage: its TM A rows and TN B rows
        uint64_t sa[TM], sb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) sa[i] = scur[wm * WTM + i * 32 + (lane & 31)];
#pragma unroll
        for (int j = 0; j < TN; ++j) sb[j] = scur[BM + wn * WTN + j * 32 + (lane & 31)];
        const uint8_t *sa_t = cur, *sb_t = cur + A_BYTES;
#pragma unroll
        for (int ks = 0; ks < FK / 64; ++ks) {
            if (kt * (FK / 64) + ks >= nsub) break;         // uniform: the K tail
            const int c = ks * 2 + (lane >> 5);               // 16-byte chunk = 32 codes
            v8i af[TM], bfr[TN];
            int sca[TM], scb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm * WTM + i * 32 + (lane & 31);
                const uint4 q = *reinterpret_cast<const uint4 *>(sa_t + r * ROW_BYTES + swz(r, c) * 16);
                af[i] = (v8i){(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
                sca[i] = (int)((sa[i] >> (8 * c)) & 0xFFu);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int r = wn * WTN + j * 32 + (lane & 31);
                const uint4 q = *reinterpret_cast<const uint4 *>(sb_t + r * ROW_BYTES + swz(r, c) * 16);
                bfr[j] = (v8i){(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
                scb[j] = (int)((sb[j] >> (8 * c)) & 0xFFu);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        af[i], bfr[j], acc[i][j], 4, 4, 0, sca[i], 0, scb[j]);
            // the single-wave MFMA interleaving strategy, as in k_gemm_nt
            // (about 2 us off the 8192x2880x5760 product)
            __builtin_amdgcn_iglp_opt(1);
        }
        // the other scale buffer was last read in the previous stage, before
        // its closing barrier; past the last stage the values go unused
        snxt[tid] = pack_scales(h);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    {
        uint32_t h[FSB / 2];
        load_scales(0, h);
        issue_stage(0, lds0);
        sc0[tid] = pack_scales(h);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
        stage(kt, lds0, lds1, sc0, sc1);
        if (kt + 1 < nk) stage(kt + 1, lds1, lds0, sc1, sc0);
    }

    // epilogue through this wave's 16 KB of the stage buffers (all reads of
    // them ended at the last barrier)
    uint8_t *ep = (wave < 4 ? lds0 : lds1) + (wave & 3) * (WTM * WTN * 2);
    store_wave_tile<TM, TN>(acc, ep, C, keep, tm * BM + wm * WTM, tn * BN + wn * WTN, M, N,
                            lane);
}

int tile_count(int64_t M, int64_t N) { return (int)(((M + BM - 1) / BM) * ((N + BN - 1) / BN)); }

Problem make_problem(const void *a, const void *bt, void *c, int64_t M, int64_t N, int64_t K)
{
    Problem p;
    p.A = (const uint16_t *)a;
    p.Bt = (const uint16_t *)bt;
    p.C = (uint16_t *)c;
    p.keep = nullptr;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.tiles = tile_count(M, N);
    return p;
}

// The epilogue stores 16-byte chunks of 8 columns: C rows must be whole chunks.
bool epilogue_ok(const void *c, int64_t N)
{
    return N % 8 == 0 && ((uintptr_t)c & 15) == 0;
}

}  // namespace

namespace fqimpl {

hipError_t launch_gemm_bf16_nt(const void *a, const void *bt, void *c, int64_t M, int64_t N,
                               int64_t K, hipStream_t stream)
{
    if (!epilogue_ok(c, N)) return hipErrorInvalidValue;
    Problem p0 = make_problem(a, bt, c, M, N, K), p1 = p0;
    p1.tiles = 0;
    hipLaunchKernelGGL(k_gemm_nt, dim3((uint32_t)p0.tiles), dim3(kThreads), 0, stream, p0, p1);
    return hipGetLastError();
}

hipError_t launch_gemm_bf16_nt_pair(const void *a0, const void *bt0, void *c0, int64_t M0,
                                    int64_t N0, int64_t K0, const void *a1, const void *bt1,
                                    void *c1, int64_t M1, int64_t N1, int64_t K1,
                                    hipStream_t stream, const void *keep0, const void *keep1)
{
    if (!epilogue_ok(c0, N0) || !epilogue_ok(c1, N1)) return hipErrorInvalidValue;
    Problem p0 = make_problem(a0, bt0, c0, M0, N0, K0);
    Problem p1 = make_problem(a1, bt1, c1, M1, N1, K1);
    p0.keep = (const uint8_t *)keep0;
    p1.keep = (const uint8_t *)keep1;
    // longer per-tile contraction first; the first problem's share of the
    // grid is padded to a multiple of the XCD count so that the second keeps
    // its XCD-contiguous tile order
    if (p1.K > p0.K) {
        const Problem t = p0;
        p0 = p1;
        p1 = t;
    }
    p0.tiles = (p0.tiles + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL(k_gemm_nt, dim3((uint32_t)(p0.tiles + p1.tiles)), dim3(kThreads), 0,
                       stream, p0, p1);
    return hipGetLastError();
}

hipError_t launch_gemm_mxfp4_nt_pair(const Fp4Operands &o0, const Fp4Operands &o1, int count,
                                     hipStream_t stream)
{
    auto mk = [](const Fp4Operands &o) {
        Fp4Problem p;
        p.A = (const uint8_t *)o.a_codes;
        p.As = (const uint8_t *)o.a_scales;
        p.B = (const uint8_t *)o.b_codes;
        p.Bs = (const uint8_t *)o.b_scales;
        p.C = (uint16_t *)o.c;
        p.keep = (const uint8_t *)o.keep;
        p.M = (int)o.M;
        p.N = (int)o.N;
        p.K = (int)o.K;
        p.tiles = tile_count(o.M, o.N);
        return p;
    };
    if (!epilogue_ok(o0.c, o0.N) || (count > 1 && !epilogue_ok(o1.c, o1.N)))
        return hipErrorInvalidValue;
    Fp4Problem p0 = mk(o0), p1 = mk(count > 1 ? o1 : o0);
    if (count < 2) {
        p1.tiles = 0;
    } else {
        if (p1.K > p0.K) {
            const Fp4Problem t = p0;
            p0 = p1;
            p1 = t;
        }
        p0.tiles = (p0.tiles + kXcds - 1) / kXcds * kXcds;
    }
    hipLaunchKernelGGL(k_gemm_mxfp4_nt, dim3((uint32_t)(p0.tiles + p1.tiles)), dim3(kThreads), 0,
                       stream, p0, p1);
    return hipGetLastError();
}

}  // namespace fqimpl
