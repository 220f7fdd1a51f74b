/*
 * fq.h -- blockwise FP4 fake quantization on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libfq.so.  Every call validates its arguments on the host, then
 * enqueues hand-written HIP kernels on the caller's stream and returns.  The
 * library allocates no device memory and keeps no state between calls other
 * than a thread-local error message; scratch memory comes from the caller's
 * workspace argument.
 *
 * Sources for the operations (cited by page title and section):
 *  - "Como o Treinamento com Quantizacao Detecta e Recupera Precisao em
 *    Inferencia de Baixa Precisao" (brainai.pro), "Detalhes tecnicos ou
 *    Implementacao": QAT fake-quantizes weights and activations in the
 *    forward pass (quantize then dequantize inside a wider type) and passes
 *    gradients through the quantizer with the straight-through estimator,
 *    exposing rounding and clipping effects.
 *  - "Aprimorando gpt-oss para Precisao e Desempenho com Treinamento
 *    Consciente a Quantizacao" (brainai.pro), "O que ha de novo", and the
 *    gpt-oss QAT tutorial (thakicloud), "NVFP4: The Next Generation": MXFP4
 *    and NVFP4 targets, NVFP4's FP8 E4M3 block scale, switching between the
 *    two formats as a one-line configuration change.
 *  - "Resumo Tecnico: TetraJet-v2" (gist.science), sec. 2.A: NVFP4 groups of
 *    16 elements with an 8-bit scale; a 128-element outer block with its own
 *    scale over 16-element inner blocks instead of a tensor-wide maximum;
 *    stochastic rounding with E[round(x)] = x in the backward pass; 1x16
 *    weight groups with the transposed weight aligned accordingly; linear
 *    layers whose activations and weights are all quantized.
 *  - Format definitions: OCP Microscaling Formats (MX) v1.0 (FP4 E2M1
 *    element, E8M0 scale 2^(floor(log2 amax) - 2)); OCP OFP8 v1.0 (E4M3,
 *    bias 7, max 448, no infinities).  Philox4x32-10: Salmon et al., "Parallel
 *    Random Numbers: As Easy as 1, 2, 3", SC'11.
 *
 * Numerics (identical, bit for bit, on every call):
 *  - E2M1 codes: bit 3 sign, magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; the sign
 *    of x is kept, so a negative value that rounds to zero is code 8 and
 *    dequantizes to -0.0.
 *  - MXFP4 block scale: E8M0 code clamp(floor(log2 amax) - 2, -127, 127) + 127
 *    (an all-zero block gets code 0).
 *  - NVFP4 outer scale s = RN(amax_outer / 2688) in FP32 (2688 = 6 * 448),
 *    amax_outer over the whole tensor (FQ_OUTER_TENSOR) or over each
 *    128-element outer block (FQ_OUTER_BLOCK128).  Block scale code
 *    e4 = E4M3_RNE_sat(RN(RN(amax_b / 6) / s)) (0 if s = 0); effective scale
 *    s_eff = RN(e4m3(e4) * s).
 *  - Scaled magnitude a = RN(|x| / s_eff), correctly rounded FP32 (0 when
 *    s_eff = 0).
 *  - FQ_ROUND_RNE: a rounds to the nearest grid value, ties to the even
 *    code, saturating at 6.  FQ_ROUND_SR: a >= 6 gives 6; otherwise with
 *    g_k <= a < g_{k+1}, T = floor((a - g_k) / (g_{k+1} - g_k) * 65536) and
 *    the element rounds up iff r16(n) < T, where r16(n) is 16-bit half
 *    (n & 1) of word ((n >> 1) & 3) of Philox4x32-10 with key (seed low word,
 *    seed high word) and counter (low word of n >> 3, high word of n >> 3,
 *    0, 0), and n is the element's row-major index in the orientation being
 *    quantized (r * cols + c for FQ_AXIS_ROW, c * rows + r for FQ_AXIS_COL).
 *  - Dequantized value y = BF16_RNE(RN(+-g * s_eff)).
 *  - A value is clipped when a > 6.
 *
 * Layouts (all row-major, contiguous):
 *  - x, y, dy, dx: BF16 [rows, cols].
 *  - FQ_AXIS_ROW (1xB groups along each row, the contiguous axis):
 *      codes [rows, cols/2] bytes (element 2j in the low nibble),
 *      scales [rows, cols/B] bytes, outer: 1 float (TENSOR) or
 *      [rows, cols/128] floats (BLOCK128).
 *  - FQ_AXIS_COL (groups of B consecutive rows in each column, i.e. 1xB
 *    groups along the rows of x^T): codes [cols, rows/2], scales
 *    [cols, rows/B], outer 1 float or [cols, rows/128] -- the layout of x^T;
 *    y stays in the layout of x.
 *
 * Pointers: x, y, dy, dx, codes and scales are device pointers aligned to
 * 16 bytes; outer is a device pointer aligned to 4 bytes; descriptors are
 * host pointers read only during the call.  The caller owns all memory.
 *
 * Asynchrony: calls return after enqueueing on `stream` (a hipStream_t, NULL
 * for the default stream).  Results are ready when the stream reaches them.
 * A call that returns an error other than FQ_ERR_DEVICE has enqueued nothing
 * and written nothing.
 *
 * Limits: 1 <= rows, cols < 2^31 and rows * cols <= 2^34 elements.
 */
#ifndef FQ_H
#define FQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FQ_OK = 0,
    FQ_ERR_NULL = 1,       /* a required pointer is NULL */
    FQ_ERR_DESC = 2,       /* unsupported descriptor combination */
    FQ_ERR_SHAPE = 3,      /* sizes out of range or not divisible by the block */
    FQ_ERR_ALIGN = 4,      /* a pointer is not aligned as documented */
    FQ_ERR_WORKSPACE = 5,  /* workspace missing or smaller than required */
    FQ_ERR_DEVICE = 6      /* a HIP launch or query failed */
} fq_status;

enum { FQ_SCALE_E8M0 = 0, FQ_SCALE_E4M3 = 1 };
enum { FQ_OUTER_NONE = 0, FQ_OUTER_TENSOR = 1, FQ_OUTER_BLOCK128 = 2 };
enum { FQ_ROUND_RNE = 0, FQ_ROUND_SR = 1 };
enum { FQ_AXIS_ROW = 0, FQ_AXIS_COL = 1 };

/* Quantization format and rounding.  Valid combinations:
 *   MXFP4: {block_size 32, FQ_SCALE_E8M0, FQ_OUTER_NONE}
 *   NVFP4: {block_size 16, FQ_SCALE_E4M3, FQ_OUTER_TENSOR or FQ_OUTER_BLOCK128}
 * with any rounding and axis.  seed is read only for FQ_ROUND_SR. */
typedef struct {
    int32_t block_size;
    int32_t scale_type;
    int32_t outer;
    int32_t rounding;
    int32_t axis;
    int32_t reserved;      /* must be 0 */
    uint64_t seed;
} fq_desc;

/* Presets: the one-line switch between the two formats.
 * fq_desc_mxfp4() = {32, E8M0, NONE, RNE, ROW, 0, seed 0}
 * fq_desc_nvfp4() = {16, E4M3, TENSOR, RNE, ROW, 0, seed 0} */
fq_desc fq_desc_mxfp4(void);
fq_desc fq_desc_nvfp4(void);

/* Bytes of workspace that fq_quantize / fq_fake_quant need for this
 * descriptor and shape: 4096 for FQ_OUTER_TENSOR (partial maxima of the
 * per-tensor reduction), 0 otherwise.  Contents need no initialization and
 * are not meaningful after the call.  Returns 0 for an invalid descriptor. */
size_t fq_workspace_size(const fq_desc *desc, int64_t rows, int64_t cols);

/* Quantize: x -> codes, scales and (NVFP4) outer scales.
 * codes, scales must be non-NULL; outer must be non-NULL for NVFP4 and is
 * ignored for MXFP4.  ws / ws_bytes: see fq_workspace_size (ws may be NULL
 * when 0 bytes are needed).  Source: the quantize half of fake quantization
 * ("Como o Treinamento ...", "Detalhes tecnicos"); format per the header. */
fq_status fq_quantize(const fq_desc *desc, const void *x_bf16, int64_t rows,
                      int64_t cols, void *codes, void *scales, float *outer,
                      void *ws, size_t ws_bytes, void *stream);

/* Dequantize: codes, scales, outer -> y [rows, cols] BF16, where rows x cols
 * is the shape of the original x and desc->axis says which layout codes and
 * scales are in: y = BF16_RNE(RN(+-g * s_eff)) per element, the value the
 * quantized element stands for.  Rounding and seed are ignored.  codes and
 * scales are required, outer for NVFP4; shape rules as fq_quantize.  Source:
 * the dequantize half of fake quantization, which brings the quantized
 * values back into the wider type the forward pass computes in ("Como o
 * Treinamento ...", "Detalhes tecnicos ou Implementacao"); for the formats,
 * OCP MX v1.0 (an element's value is its E2M1 value times the block scale)
 * and, for NVFP4, the E4M3 block scale times the FP32 outer scale
 * ("Resumo Tecnico: TetraJet-v2", sec. 2.A). */
fq_status fq_dequantize(const fq_desc *desc, const void *codes, const void *scales,
                        const float *outer, int64_t rows, int64_t cols,
                        void *y_bf16, void *stream);

/* Fake quantization: y = dequantize(quantize(x)) in one pass over x.
 * y must be non-NULL; codes, scales and outer may each be NULL to skip that
 * output.  Source: "Como o Treinamento ...", "Detalhes tecnicos" (fake
 * quantization in the forward pass); TetraJet-v2 sec. 2.A for the double
 * block and stochastic rounding. */
fq_status fq_fake_quant(const fq_desc *desc, const void *x_bf16, int64_t rows,
                        int64_t cols, void *y_bf16, void *codes, void *scales,
                        float *outer, void *ws, size_t ws_bytes, void *stream);

/* Straight-through estimator with clipping: dx = dy where the forward did
 * not clip x (a <= 6), else +0.  a is recomputed from x and the forward's
 * stored scales (and outer scales) in the forward's layout (desc->axis).
 * Source: "Como o Treinamento ...", "Detalhes tecnicos" (gradients through
 * the quantizer by STE; clipping effects). */
fq_status fq_ste_backward(const fq_desc *desc, const void *x_bf16,
                          const void *scales, const float *outer,
                          const void *dy_bf16, int64_t rows, int64_t cols,
                          void *dx_bf16, void *stream);

/* fq_fake_quant for callers that cannot allocate or pass a workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation and outputs, with the per-tensor
 * maximum's partials (the only scratch any format needs, at most 4096 bytes
 * whatever the shape) in a 4 KB device array the library owns, one per GPU,
 * instead of ws.  The call allocates nothing.  Calls on one GPU share that
 * array: calls that overlap on one GPU (different streams, or different
 * threads) race and must be serialized by the caller.  Arguments and errors
 * otherwise as fq_fake_quant; FQ_ERR_DEVICE if the array's address cannot be
 * looked up on the current device. */
fq_status fq_fake_quant_noalloc(const fq_desc *desc, const void *x_bf16, int64_t rows,
                                int64_t cols, void *y_bf16, void *codes, void *scales,
                                float *outer, void *stream);

/* Fake quantization that also writes the STE keep mask: as fq_fake_quant,
 * plus keep [rows, cols / 8] uint8 in the layout of x (row-major, whatever
 * desc->axis is): bit (c mod 8) of byte (r, c / 8) is 1 where element (r, c)
 * was kept (a = RN(|x| / s_eff) <= 6) and 0 where the forward clipped it.
 * The backward then needs neither x nor the scales (fq_ste_backward_mask):
 * the clipped STE reads 2 B of dy and 1/8 B of mask per element instead of
 * 2 B of x plus the scales.  cols must be a multiple of 8; keep must be
 * non-NULL, 16-byte aligned, and must not overlap the other buffers.  Errors
 * as fq_fake_quant.  Source: TetraJet-v2 sec. 2.A (the backward passes
 * gradients through the quantizer where it did not clip); "Como o
 * Treinamento ...", "Detalhes tecnicos" (STE, clipping effects). */
fq_status fq_fake_quant_mask(const fq_desc *desc, const void *x_bf16, int64_t rows,
                             int64_t cols, void *y_bf16, void *codes, void *scales,
                             float *outer, void *keep, void *ws, size_t ws_bytes,
                             void *stream);

/* Fake quantization of the random Hadamard rotation of x along the
 * quantization axis, in one pass: y = dequantize(quantize(H x)), codes and
 * scales of H x.  H is blockwise H_n (n = rht_block, 16 or 128) with the
 * Philox sign vector of rht_seed, exactly as fq_hadamard computes it
 * (including the BF16 rounding of the rotated values), so the result equals
 * fq_fake_quant applied to fq_hadamard's output.  desc: MXFP4 or NVFP4
 * FQ_OUTER_BLOCK128 (the per-tensor scale would need the rotated tensor's
 * maximum first), either axis, RNE or SR; the quantized axis a multiple of
 * rht_block.  y required; codes, scales, outer optional.  Source: "Resumo
 * Tecnico: TetraJet-v2", sec. 2.C (the rotation ahead of the backward's FP4
 * quantization). */
fq_status fq_fake_quant_rht(const fq_desc *desc, const void *x_bf16, int64_t rows, int64_t cols,
                            int32_t rht_block, uint64_t rht_seed, void *y_bf16, void *codes,
                            void *scales, float *outer, void *stream);

/* Clipped straight-through estimator from a keep mask written by
 * fq_fake_quant_mask: dx = dy where the element's keep bit is set, else +0.
 * keep [rows, cols / 8] (layout above), dy and dx [rows, cols] BF16, all
 * device pointers, 16-byte aligned; dx may alias dy.  rows >= 1, cols >= 8,
 * cols a multiple of 8.  Format independent.  Source: as fq_ste_backward. */
fq_status fq_ste_backward_mask(const void *keep, const void *dy_bf16, int64_t rows,
                               int64_t cols, void *dx_bf16, void *stream);

/* Workspace for fq_qlinear_fwd: the dequantized X_hat [M, K] BF16 at offset
 * 0, the dequantized and transposed W_hat^T [N, K] BF16 at offset
 * round_up(M * K * 2, 256), then 8192 bytes of reduction scratch.  When both
 * descriptors are MXFP4, the operands stay encoded instead: X's codes [M, K/2] at 0, X's E8M0 scales [M, K/32] at
 * c1 = round_up(M * K / 2, 256), W's codes in the transposed layout [N, K/2]
 * at c2 = c1 + round_up(M * K / 32, 256), W's scales [N, K/32] at
 * c2 + round_up(N * K / 2, 256) (same total size).  0 for dimensions outside
 * the limits of fq_qlinear_fwd. */
size_t fq_qlinear_workspace_size(const fq_desc *desc_x, const fq_desc *desc_w,
                                 int64_t M, int64_t K, int64_t N);

/* QAT linear forward: Y [M, N] BF16 = FQ(X) [M, K] x FQ(W) [K, N] with FP32
 * accumulation on the matrix cores.  X is quantized in groups along K (its
 * rows: desc_x->axis must be FQ_AXIS_ROW), W in groups along K (its
 * columns: desc_w->axis must be FQ_AXIS_COL), so both operands are blocked
 * along the contraction.  Shapes: M, N >= 1; K a multiple of 64 (the
 * matrix-core kernels step through K 64 elements at a time and have no
 * partial step; this also covers both block sizes), and of 128 for
 * FQ_OUTER_BLOCK128; N a multiple of 8 (W is quantized along its columns,
 * whose kernels move 8 columns at a time); M, K, N < 2^31 and M * K, K * N
 * and M * N <= 2^34.
 * Otherwise FQ_ERR_SHAPE.
 * Source: gpt-oss QAT tutorial, "NVFP4: The Next Generation"
 * (weight-activation quantization of the MLP); TetraJet-v2 sec. 2 (NVFP4
 * activations and weights in every linear layer).  MXFP4 x MXFP4 multiplies the E2M1 codes with their E8M0 block scales on the scaled FP4
 * matrix cores (OCP Microscaling v1.0 block scaling), which is the same
 * product of the same dequantized values. */
fq_status fq_qlinear_fwd(const fq_desc *desc_x, const fq_desc *desc_w,
                         const void *x_bf16, const void *w_bf16, int64_t M,
                         int64_t K, int64_t N, void *y_bf16, void *ws,
                         size_t ws_bytes, void *stream);

/* Random Hadamard transform: y = BF16_RNE(RN32(c_n * H_n (s o x))) in
 * blocks of n = 16 or 128 consecutive elements along `axis` (FQ_AXIS_ROW:
 * along each row; FQ_AXIS_COL: down each column), where H_n is the Hadamard
 * matrix in Sylvester order applied by radix-2 FP32 butterflies (half-widths
 * 1, 2, ..., n/2; a pair (a, b) becomes (a + b, a - b)), c_n the FP32 value
 * nearest to 1/sqrt(n), and s_j = -1 where bit (j mod 128) of
 * Philox4x32-10(key = seed, counter = (j / 128, 0, 0, 0)) is set (bit t of
 * output word w counts as bit 32w + t), j the position along the axis.
 * x, y: device [rows, cols] BF16, 16-byte aligned, not overlapping.  The
 * transformed axis must be a multiple of n; FQ_AXIS_COL needs cols % 8 == 0.
 * Source: "Resumo Tecnico: TetraJet-v2", sec. 2.C (OutControl: a random
 * Hadamard transform on the backward's products spreads outlier energy). */
fq_status fq_hadamard(const void *x_bf16, int64_t rows, int64_t cols, int32_t axis,
                      int32_t block, uint64_t seed, void *y_bf16, void *stream);

/* Workspace for fq_qlinear_bwd (internal layout; the size depends only on
 * the arguments). */
size_t fq_qlinear_bwd_workspace_size(const fq_desc *desc_x, const fq_desc *desc_w,
                                     const fq_desc *desc_g, int32_t rht_block, int64_t M,
                                     int64_t K, int64_t N);

/* QAT linear backward of fq_qlinear_fwd (Y = FQ(X) x FQ(W), X [M, K],
 * W [K, N]), given dY [M, N]:
 *   dX [M, K] = STE_X( Q(dY) x Q(W_hat)^T ),  Q along N for both operands,
 *   dW [K, N] = STE_W( Q(X_hat)^T x Q(dY) ),  Q along M for both operands,
 * where X_hat = FQ(X, desc_x) and W_hat = FQ(W, desc_w) are the forward's
 * fake-quantized operands (recomputed here), Q quantizes with desc_g's
 * format and rounding along the contraction axis of each product, and
 * STE_X / STE_W pass a gradient entry where the forward did not clip that
 * entry of X / W (a <= 6) and write +0 where it did.  The four Q draws use
 * Philox keys desc_g->seed + 0 (dY along N), + 1 (W_hat along N), + 2 (X_hat
 * along M), + 3 (dY along M); desc_g->axis is ignored.  rht_block = 16 or
 * 128 first rotates both operands of each product along its contraction axis
 * by the random Hadamard transform of fq_hadamard with seed rht_seed (which
 * cancels in the exact product); 0 leaves them as they are (with an MXFP4 or
 * double-block desc_g the rotation runs inside the quantizers, as in
 * fq_fake_quant_rht).  Products accumulate in FP32 on the matrix cores and are
 * rounded to BF16 before the STE, which is applied as the product is stored.
 * With an MXFP4 desc_g both products run on the scaled FP4 matrix cores from
 * the gradient operands' codes and E8M0 scales.
 * Shapes: K a multiple of 8 and of desc_x's and desc_w's block sizes (128
 * for FQ_OUTER_BLOCK128); M and N multiples of 64 and of desc_g's block size
 * (128 for FQ_OUTER_BLOCK128) and of rht_block; desc_x->axis FQ_AXIS_ROW,
 * desc_w->axis FQ_AXIS_COL as in the forward.
 * Pointers x, w, dy, dx, dw, ws: device, 16-byte aligned, caller-owned; ws
 * at least fq_qlinear_bwd_workspace_size bytes.  Errors as fq_qlinear_fwd.
 * Source: TetraJet-v2, sec. 2.A (the backward computes on the aligned X_hat,
 * with stochastic rounding so that E[round(x)] = x, and 1x16 weight groups
 * realigned for the transposed weight) and sec. 2.C (random Hadamard
 * transform of the backward's products); "Como o Treinamento ...",
 * "Detalhes tecnicos" (gradients pass the quantizer by STE, clipping
 * effects). */
fq_status fq_qlinear_bwd(const fq_desc *desc_x, const fq_desc *desc_w,
                         const fq_desc *desc_g, int32_t rht_block, uint64_t rht_seed,
                         const void *x_bf16, const void *w_bf16, const void *dy_bf16,
                         int64_t M, int64_t K, int64_t N, void *dx_bf16, void *dw_bf16,
                         void *ws, size_t ws_bytes, void *stream);

/* ---- TetraJet-v2 OsciReset ("Resumo Tecnico: TetraJet-v2", sec. 2.B) ----
 * Per-element state of n weights, all device arrays the caller owns: w_prev
 * and dist_m, dist_q FP32 [n], q_prev BF16 [n].  w is the FP32 master weight,
 * q the BF16 fake-quantized weight the forward pass used.  n >= 4, n a
 * multiple of 4; every pointer 16-byte aligned (q, q_prev: 8-byte).
 *
 * fq_osci_track: one training step.  dist_m += |w - w_prev| and dist_q +=
 * |q - q_prev| (FP32, one rounding per operation), then w_prev = w and
 * q_prev = q.  first != 0 starts the trajectory: records w and q and zeroes
 * the distances (no memset: safe inside a captured graph). */
fq_status fq_osci_track(const float *w, const void *q_bf16, float *w_prev, void *q_prev_bf16,
                        float *dist_m, float *dist_q, int64_t n, int32_t first, void *stream);

/* fq_osci_reset: the check, called when the learning rate is low.  The
 * oscillation risk is dist_q / dist_m; an element with dist_q > RN(tau *
 * dist_m) is reset, all others keep w.  Then every element starts a new
 * window: w_prev = w, q_prev = q, distances 0.  tau is the risk threshold
 * (finite, >= 0).  w, q and the state are [rows, cols] row-major (n =
 * rows * cols), cols a multiple of 4.
 * target FQ_OSCI_BIN_CENTRE (sec. 2.B, "Mecanismo": the master weight goes
 * to the centre of its current quantization bin): w = sign * RN(c_m * s_eff)
 * for the element's current E2M1 code (sign, magnitude m) and effective
 * block scale s_eff, read from codes / scales / outer, the fq_quantize or
 * fq_fake_quant outputs of the quantization that gave q, in desc's format
 * and axis layout (rows x cols is the shape of that quantization's input).
 * c_m is the centre of the interval of scaled magnitudes that round to grid
 * value g_m: 0, 0.5, 1, 1.5, 2.125, 3, 4.25, 6 for g = 0, 0.5, 1, 1.5, 2, 3,
 * 4, 6 (the bins of 2 and 4, [1.75, 2.5] and [3.5, 5], are lopsided; the top
 * bin, from 5, is read as closing at 7, midway to 8, the next value of the
 * E2M1 exponent progression, so its centre is 6).  desc, codes, scales
 * (16-byte aligned) are required, outer (4-byte aligned) for NVFP4; desc's
 * shape rules are those of fq_quantize.
 * target FQ_OSCI_GRID_VALUE: w = q (its quantized value); desc, codes,
 * scales and outer are not read and may be NULL. */
enum { FQ_OSCI_BIN_CENTRE = 0, FQ_OSCI_GRID_VALUE = 1 };
fq_status fq_osci_reset(const fq_desc *desc, float *w, const void *q_bf16, const void *codes,
                        const void *scales, const float *outer, int64_t rows, int64_t cols,
                        float *w_prev, void *q_prev_bf16, float *dist_m, float *dist_q,
                        float tau, int32_t target, void *stream);

/* ---- TetraJet-v2 static outlier-channel retention (sec. 2.C) ----
 * Calibration: fq_channel_absmax folds max |x[:, c]| of a BF16 [rows, cols]
 * tensor into amax [cols] (uint32, the BF16 magnitude bits; zero it once before
 * the first batch), by integer atomic maximum, so the result does not depend
 * on order.  cols a multiple of 8; x 16-byte and amax 4-byte aligned. */
fq_status fq_channel_absmax(const void *x_bf16, int64_t rows, int64_t cols, uint32_t *amax,
                            void *stream);

/* Selection: the k channels with the largest amax (ties: lower index first)
 * are retained.  Writes retain [cols / 8] (bit c mod 8 of byte c / 8 set for a
 * retained channel) and chan_scale [cols] FP32 = amax_c / 448 (the largest
 * E4M3 value; 0 for other channels).  0 <= k <= cols, cols a multiple of 8. */
fq_status fq_select_channels(const uint32_t *amax, int64_t cols, int64_t k, void *retain,
                             float *chan_scale, void *stream);

/* Fake quantization with retained channels, along either axis: the columns
 * of x whose retain bit is set (the activation's channels) are FP8 E4M3
 * fake-quantized under chan_scale (|x| / s in FP32, nearest-even, saturating
 * at 448, times s, sign kept; s = 0 gives +-0) and carry FP4 code 0; every
 * FP4 block, 128-element outer and per-tensor maximum is taken over the other
 * elements only.  That is the plain fake quantization of x with the retained
 * columns set to +0, the FP8 values in their place.  FQ_AXIS_ROW: the
 * retained columns drop out of the 1xB groups they share; FQ_AXIS_COL: every
 * group of a retained column is empty.  desc: any format, rounding and axis;
 * cols a multiple of 8; y required, codes, scales, outer optional (as
 * fq_fake_quant); retain and chan_scale as written by fq_select_channels,
 * chan_scale 16-byte aligned; ws / ws_bytes as fq_fake_quant (per-tensor
 * NVFP4: 4096 bytes).  Source: "Resumo Tecnico: TetraJet-v2", sec. 2.C
 * (OutControl, "Retencao Estatica de Outliers": the top p % channels stay in
 * FP8 in the forward and the backward pass, the rest in FP4). */
fq_status fq_fake_quant_retain(const fq_desc *desc, const void *x_bf16, int64_t rows,
                               int64_t cols, void *y_bf16, void *codes, void *scales,
                               float *outer, const void *retain, const float *chan_scale,
                               void *ws, size_t ws_bytes, void *stream);

/* fq_qlinear_fwd with the activation's retained channels (columns of X, as
 * fq_fake_quant_retain along the row axis) kept in FP8: Y = FQ_retain(X) x
 * FQ(W) on the BF16 matrix cores (whatever the formats).  Arguments and
 * workspace as fq_qlinear_fwd, plus retain [K/8] and chan_scale [K]; K a
 * multiple of 8.  Source: "Resumo Tecnico: TetraJet-v2", sec. 2.C (forward
 * pass). */
fq_status fq_qlinear_fwd_retain(const fq_desc *desc_x, const fq_desc *desc_w, const void *x_bf16,
                                const void *w_bf16, int64_t M, int64_t K, int64_t N,
                                const void *retain, const float *chan_scale, void *y_bf16,
                                void *ws, size_t ws_bytes, void *stream);

/* fq_qlinear_bwd (without the rotation) with the activation's retained
 * channels kept in FP8: X_hat is fq_fake_quant_retain of X along the row
 * axis, X_hat's quantization along M for dW keeps the same channels in FP8
 * (fq_fake_quant_retain along the column axis with desc_g's format, rounding
 * and key seed + 2), and STE_X passes a retained entry where |x| / s <= 448
 * (the FP8 format's clip).  Both products run on the BF16 matrix cores.
 * Arguments and workspace as fq_qlinear_bwd with rht_block = 0, plus retain
 * [K/8] and chan_scale [K]; K a multiple of 8.  Source: "Resumo Tecnico:
 * TetraJet-v2", sec. 2.C (forward and backward pass). */
fq_status fq_qlinear_bwd_retain(const fq_desc *desc_x, const fq_desc *desc_w,
                                const fq_desc *desc_g, const void *x_bf16, const void *w_bf16,
                                const void *dy_bf16, int64_t M, int64_t K, int64_t N,
                                const void *retain, const float *chan_scale, void *dx_bf16,
                                void *dw_bf16, void *ws, size_t ws_bytes, void *stream);

/* Static description of a status code. */
const char *fq_status_string(fq_status s);

/* Message of the last error on the calling thread ("" if none). */
const char *fq_last_error(void);

/* Library version, e.g. "0.1.0". */
const char *fq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FQ_H */
