// fq_internal.h -- launchers shared between the C-ABI layer and the kernels.
// Arguments are validated by the caller (fq_api.cpp); launchers only map the
// problem onto a grid and enqueue on `stream`.  Each returns hipSuccess or
// the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fqimpl {

enum { FMT_MX = 0, FMT_NVT = 1, FMT_NV128 = 2 };

// Number of partial maxima the per-tensor reduction writes (4 bytes each).
constexpr uint32_t kAbsmaxPartials = 1024;

struct QuantArgs {
    int fmt;              // FMT_*
    int sr;               // 0 = round to nearest even, 1 = stochastic
    int col;              // 0 = groups along rows of x, 1 = along columns
    uint64_t seed;
    const void *x;        // BF16 [R, C]
    int64_t R, C;
    void *y;              // BF16 [R, C] or null
    void *yt;             // column axis only: BF16 [C, R] (y transposed) or null
    void *codes;          // or null
    void *scales;         // or null
    float *outer;         // or null
    void *keep = nullptr; // uint8 [R, C/8] STE keep mask in the layout of x, or null
    int rht_n = 0;        // 16 / 128: quantize the random Hadamard rotation of x along
    uint64_t rht_seed = 0; //  the quantization axis (not with the per-tensor format)
    uint32_t *partials;   // kAbsmaxPartials words (NV per-tensor only)
    bool cached_outputs;  // ordinary stores (outputs re-read right away) instead of streaming
    // column axis only: retained FP8 channels (columns of x; bit mask [C/8])
    // and their FP32 scales [C], or null
    const void *retain = nullptr;
    const float *chan_scale = nullptr;
};

// Partial maxima of |x| for the per-tensor NVFP4 scale; with retain (bit
// c mod 8 of byte c / 8 for column c of a row of `cols` elements) the
// retained columns are left out.
hipError_t launch_absmax(const void *x, int64_t n_elems, uint32_t *partials,
                         uint32_t *npart_out, hipStream_t stream,
                         const void *retain = nullptr, int64_t cols = 0);
// The partial maxima of two tensors in one launch (no retained columns).
hipError_t launch_absmax_pair(const void *x0, int64_t n0, uint32_t *partials0, uint32_t *npart0,
                              const void *x1, int64_t n1, uint32_t *partials1, uint32_t *npart1,
                              hipStream_t stream);
hipError_t launch_quant(const QuantArgs &a, uint32_t npart, hipStream_t stream);
hipError_t launch_dequant(int fmt, int col, const void *codes, const void *scales,
                          const float *outer, int64_t R, int64_t C, void *y,
                          hipStream_t stream);
// dx = dy where the keep bit (bit c mod 8 of byte (r, c / 8)) is set, else +0.
hipError_t launch_ste_mask(const void *keep, const void *dy, int64_t R, int64_t C, void *dx,
                           hipStream_t stream);
hipError_t launch_ste(int fmt, int col, const void *x, const void *scales,
                      const float *outer, const void *dy, int64_t R, int64_t C,
                      void *dx, hipStream_t stream);
// MXFP4 product on the scaled FP4 matrix cores: C [M, N] BF16 = A . B^T with
// A given as E2M1 codes [M, K/2] and E8M0 scales [M, K/32], B as codes
// [N, K/2] and scales [N, K/32]; K a multiple of 64.
struct Fp4Operands {
    const void *a_codes, *a_scales, *b_codes, *b_scales;
    void *c;
    int64_t M, N, K;
    const void *keep = nullptr;   // optional STE keep mask of c (elements zeroed where clear)
};
hipError_t launch_gemm_mxfp4_nt_pair(const Fp4Operands &o0, const Fp4Operands &o1, int count,
                                     hipStream_t stream);

// Random Hadamard transform of x [R, C] in blocks of n (16 or 128) along the
// rows (col = 0) or the columns (col = 1) into y (same layout).
hipError_t launch_hadamard(const void *x, int64_t R, int64_t C, int col, int n, uint64_t seed,
                           void *y, bool cached, hipStream_t stream);
hipError_t launch_gemm_bf16_nt(const void *a, const void *bt, void *c, int64_t M,
                               int64_t N, int64_t K, hipStream_t stream);
// Two independent products C0 = A0 * Bt0^T and C1 = A1 * Bt1^T in one launch.
// keep0 / keep1: optional STE keep masks of c0 / c1 (bit n mod 8 of byte n / 8
// for element n of C in row-major order); clear bits store +0.
hipError_t launch_gemm_bf16_nt_pair(const void *a0, const void *bt0, void *c0, int64_t M0,
                                    int64_t N0, int64_t K0, const void *a1, const void *bt1,
                                    void *c1, int64_t M1, int64_t N1, int64_t K1,
                                    hipStream_t stream, const void *keep0 = nullptr,
                                    const void *keep1 = nullptr);

// TetraJet-v2 sec. 2.B / 2.C (fq_outcontrol.hip).  n is a multiple of 4.
hipError_t launch_osci_track(const float *w, const void *q, float *w_prev, void *q_prev,
                             float *dist_m, float *dist_q, int64_t n, int first,
                             hipStream_t stream);
struct OsciResetArgs {
    float *w;                // FP32 [R, C] master weight (n = R * C elements)
    const void *q;           // BF16 [R, C] quantized weight
    float *w_prev;
    void *q_prev;
    float *dist_m, *dist_q;
    int64_t n, R, C;
    float tau;
    bool grid_target;        // reset to q instead of the bin centre
    int fmt;                 // FMT_* of the quantization that gave q (bin-centre target)
    bool col;                // its axis
    const void *codes, *scales;
    const float *outer;
};
hipError_t launch_osci_reset(const OsciResetArgs &a, hipStream_t stream);
hipError_t launch_channel_absmax(const void *x, int64_t R, int64_t C, uint32_t *amax,
                                 hipStream_t stream);
hipError_t launch_select_channels(const uint32_t *amax, int64_t C, int64_t k, void *retain,
                                  float *chan_scale, hipStream_t stream);
// Row-axis fake quantization with retained FP8 channels (any format; the
// per-tensor one takes `npart` partial maxima over the other channels).
struct RetainArgs {
    int fmt;                 // FMT_*
    int sr;
    uint64_t seed;
    const void *x;           // BF16 [R, C]
    int64_t R, C;
    const void *retain;      // uint8 [C/8] channel bit mask
    const float *chan_scale; // FP32 [C]
    void *y, *codes, *scales;
    float *outer;
    void *keep = nullptr;          // STE keep mask [R, C/8] or null
    const uint32_t *partials = nullptr;
    uint32_t npart = 0;
    bool cached_outputs = false;
};
hipError_t launch_quant_retain(const RetainArgs &a, hipStream_t stream);

}  // namespace fqimpl
