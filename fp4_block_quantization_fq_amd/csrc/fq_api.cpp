// fq_api.cpp -- the C ABI of libfq.so (declared in include/fq.h).
//
// Every entry point validates its arguments completely before touching the
// device: a rejected call enqueues nothing and writes nothing.  Accepted calls
// enqueue kernels on the caller's stream and return; launch failures are
// reported as FQ_ERR_DEVICE.  No exception crosses the boundary.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "fq.h"
#include "fq_internal.h"

namespace {

thread_local char g_err[512] = "";

fq_status fail(fq_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

fq_status ok()
{
    g_err[0] = '\0';
    return FQ_OK;
}

constexpr int64_t kMaxElems = int64_t(1) << 34;
// every dimension fits the kernels' 32-bit row/column arguments and the
// products' int tile arithmetic
constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;

struct Fmt {
    int fmt;   // fqimpl::FMT_*
    int B;     // block size
};

fq_status check_desc(const fq_desc *d, Fmt *out, const char *name)
{
    if (!d) return fail(FQ_ERR_NULL, "%s is NULL", name);
    if (d->reserved != 0) return fail(FQ_ERR_DESC, "%s->reserved must be 0", name);
    if (d->rounding != FQ_ROUND_RNE && d->rounding != FQ_ROUND_SR)
        return fail(FQ_ERR_DESC, "%s->rounding=%d is not FQ_ROUND_RNE/SR", name, d->rounding);
    if (d->axis != FQ_AXIS_ROW && d->axis != FQ_AXIS_COL)
        return fail(FQ_ERR_DESC, "%s->axis=%d is not FQ_AXIS_ROW/COL", name, d->axis);
    if (d->block_size == 32 && d->scale_type == FQ_SCALE_E8M0 && d->outer == FQ_OUTER_NONE) {
        *out = {fqimpl::FMT_MX, 32};
        return FQ_OK;
    }
    if (d->block_size == 16 && d->scale_type == FQ_SCALE_E4M3) {
        if (d->outer == FQ_OUTER_TENSOR) {
            *out = {fqimpl::FMT_NVT, 16};
            return FQ_OK;
        }
        if (d->outer == FQ_OUTER_BLOCK128) {
            *out = {fqimpl::FMT_NV128, 16};
            return FQ_OK;
        }
    }
    return fail(FQ_ERR_DESC,
                "%s: unsupported format {block_size=%d, scale_type=%d, outer=%d}; valid: "
                "MXFP4 {32, E8M0, NONE}, NVFP4 {16, E4M3, TENSOR|BLOCK128}",
                name, d->block_size, d->scale_type, d->outer);
}

fq_status check_shape(const Fmt &f, int axis, int64_t R, int64_t C)
{
    if (R < 1 || C < 1) return fail(FQ_ERR_SHAPE, "rows=%lld cols=%lld must be >= 1",
                                    (long long)R, (long long)C);
    if (R > kMaxDim || C > kMaxDim || R * C > kMaxElems)
        return fail(FQ_ERR_SHAPE, "rows=%lld cols=%lld: each must be below 2^31 and rows*cols at most 2^34", (long long)R,
                    (long long)C);
    const int64_t q = (axis == FQ_AXIS_ROW) ? C : R;    // quantized axis length
    const char *qn = (axis == FQ_AXIS_ROW) ? "cols" : "rows";
    if (q % f.B != 0)
        return fail(FQ_ERR_SHAPE, "%s=%lld must be a multiple of the block size %d", qn,
                    (long long)q, f.B);
    if (f.fmt == fqimpl::FMT_NV128 && q % 128 != 0)
        return fail(FQ_ERR_SHAPE, "%s=%lld must be a multiple of the 128-element outer block",
                    qn, (long long)q);
    if (axis == FQ_AXIS_COL && C % 8 != 0)
        return fail(FQ_ERR_SHAPE, "cols=%lld must be a multiple of 8 for FQ_AXIS_COL",
                    (long long)C);
    return FQ_OK;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

fq_status check_ptr(const void *p, const char *name, bool required, uintptr_t align = 16)
{
    if (!p) {
        if (required) return fail(FQ_ERR_NULL, "%s is NULL", name);
        return FQ_OK;
    }
    if (!aligned(p, align))
        return fail(FQ_ERR_ALIGN, "%s=%p is not %u-byte aligned", name, p, (unsigned)align);
    return FQ_OK;
}

size_t quant_ws(const Fmt &f)
{
    return f.fmt == fqimpl::FMT_NVT ? fqimpl::kAbsmaxPartials * sizeof(uint32_t) : 0;
}

fq_status device_status(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(FQ_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

#define FQ_TRY(expr)                       \
    do {                                   \
        fq_status _s = (expr);             \
        if (_s != FQ_OK) return _s;        \
    } while (0)

// Shared body of fq_quantize / fq_fake_quant once arguments are checked.
fq_status run_quant(const Fmt &f, const fq_desc *d, const void *x, int64_t R, int64_t C,
                    void *y, void *codes, void *scales, float *outer, void *ws,
                    hipStream_t st, bool cached = false, void *keep = nullptr, int rht_n = 0,
                    uint64_t rht_seed = 0, int64_t npart_given = -1)
{
    fqimpl::QuantArgs a;
    a.fmt = f.fmt;
    a.sr = d->rounding == FQ_ROUND_SR;
    a.col = d->axis == FQ_AXIS_COL;
    a.seed = d->seed;
    a.x = x;
    a.R = R;
    a.C = C;
    a.y = y;
    a.codes = codes;
    a.scales = scales;
    a.outer = (f.fmt == fqimpl::FMT_MX) ? nullptr : outer;
    a.yt = nullptr;
    a.partials = (uint32_t *)ws;
    a.keep = keep;
    a.rht_n = rht_n;
    a.rht_seed = rht_seed;
    a.cached_outputs = cached;
    // npart_given >= 0: the per-tensor partial maxima are already in ws
    uint32_t npart = npart_given >= 0 ? (uint32_t)npart_given : 0u;
    if (f.fmt == fqimpl::FMT_NVT && npart_given < 0) {
        hipError_t e = fqimpl::launch_absmax(x, R * C, a.partials, &npart, st);
        if (e != hipSuccess) return device_status(e, "tensor absmax launch");
    }
    return device_status(fqimpl::launch_quant(a, npart, st), "quantize launch");
}

}  // namespace

extern "C" {

fq_desc fq_desc_mxfp4(void)
{
    fq_desc d;
    std::memset(&d, 0, sizeof(d));
    d.block_size = 32;
    d.scale_type = FQ_SCALE_E8M0;
    d.outer = FQ_OUTER_NONE;
    d.rounding = FQ_ROUND_RNE;
    d.axis = FQ_AXIS_ROW;
    return d;
}

fq_desc fq_desc_nvfp4(void)
{
    fq_desc d;
    std::memset(&d, 0, sizeof(d));
    d.block_size = 16;
    d.scale_type = FQ_SCALE_E4M3;
    d.outer = FQ_OUTER_TENSOR;
    d.rounding = FQ_ROUND_RNE;
    d.axis = FQ_AXIS_ROW;
    return d;
}

size_t fq_workspace_size(const fq_desc *desc, int64_t rows, int64_t cols)
{
    (void)rows;
    (void)cols;
    Fmt f;
    if (check_desc(desc, &f, "desc") != FQ_OK) return 0;
    return quant_ws(f);
}

fq_status fq_quantize(const fq_desc *desc, const void *x_bf16, int64_t rows, int64_t cols,
                      void *codes, void *scales, float *outer, void *ws, size_t ws_bytes,
                      void *stream)
{
    Fmt f;
    FQ_TRY(check_desc(desc, &f, "desc"));
    FQ_TRY(check_shape(f, desc->axis, rows, cols));
    FQ_TRY(check_ptr(x_bf16, "x", true));
    FQ_TRY(check_ptr(codes, "codes", true));
    FQ_TRY(check_ptr(scales, "scales", true));
    if (f.fmt != fqimpl::FMT_MX) FQ_TRY(check_ptr(outer, "outer", true, 4));
    const size_t need = quant_ws(f);
    if (need) {
        FQ_TRY(check_ptr(ws, "ws", true));
        if (ws_bytes < need)
            return fail(FQ_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, need);
    }
    return run_quant(f, desc, x_bf16, rows, cols, nullptr, codes, scales, outer, ws,
                     (hipStream_t)stream);
}

fq_status fq_dequantize(const fq_desc *desc, const void *codes, const void *scales,
                        const float *outer, int64_t rows, int64_t cols, void *y_bf16,
                        void *stream)
{
    Fmt f;
    FQ_TRY(check_desc(desc, &f, "desc"));
    FQ_TRY(check_shape(f, desc->axis, rows, cols));
    FQ_TRY(check_ptr(codes, "codes", true));
    FQ_TRY(check_ptr(scales, "scales", true));
    if (f.fmt != fqimpl::FMT_MX) FQ_TRY(check_ptr(outer, "outer", true, 4));
    FQ_TRY(check_ptr(y_bf16, "y", true));
    return device_status(
        fqimpl::launch_dequant(f.fmt, desc->axis == FQ_AXIS_COL, codes, scales,
                               f.fmt == fqimpl::FMT_MX ? nullptr : outer, rows, cols, y_bf16,
                               (hipStream_t)stream),
        "dequantize launch");
}

fq_status fq_fake_quant(const fq_desc *desc, const void *x_bf16, int64_t rows, int64_t cols,
                        void *y_bf16, void *codes, void *scales, float *outer, void *ws,
                        size_t ws_bytes, void *stream)
{
    Fmt f;
    FQ_TRY(check_desc(desc, &f, "desc"));
    FQ_TRY(check_shape(f, desc->axis, rows, cols));
    FQ_TRY(check_ptr(x_bf16, "x", true));
    FQ_TRY(check_ptr(y_bf16, "y", true));
    FQ_TRY(check_ptr(codes, "codes", false));
    FQ_TRY(check_ptr(scales, "scales", false));
    FQ_TRY(check_ptr(outer, "outer", false, 4));
    const size_t need = quant_ws(f);
    if (need) {
        FQ_TRY(check_ptr(ws, "ws", true));
        if (ws_bytes < need)
            return fail(FQ_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, need);
    }
    return run_quant(f, desc, x_bf16, rows, cols, y_bf16, codes, scales, outer, ws,
                     (hipStream_t)stream);
}

}  // extern "C"

// ---- the entry point that allocates nothing --------------------------------
// The per-tensor maximum's partials live in this library-owned device array
// instead of a caller workspace.  Each GPU holds its own copy (allocated with
// the code object, kept until the process ends); its address on a device is
// looked up once, with that device current, and only that address is ever
// handed to kernels.  Nothing in it needs clearing: the maximum pass writes
// every partial the quantizer then reads.  Calls that overlap on one GPU share
// it and race.
namespace {

constexpr size_t kStaticScratchBytes = fqimpl::kAbsmaxPartials * sizeof(uint32_t);   // 4 KB
static __device__ __align__(256) uint32_t scratch[fqimpl::kAbsmaxPartials];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];          // per device, null until looked up

fq_status device_scratch(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(FQ_ERR_DEVICE, "device %d beyond the %d this library tracks", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return device_status(e, "scratch symbol lookup");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return FQ_OK;
}

}  // namespace

extern "C" {

fq_status fq_fake_quant_noalloc(const fq_desc *desc, const void *x_bf16, int64_t rows,
                                int64_t cols, void *y_bf16, void *codes, void *scales,
                                float *outer, void *stream)
{
    Fmt f;
    FQ_TRY(check_desc(desc, &f, "desc"));
    FQ_TRY(check_shape(f, desc->axis, rows, cols));
    FQ_TRY(check_ptr(x_bf16, "x", true));
    FQ_TRY(check_ptr(y_bf16, "y", true));
    FQ_TRY(check_ptr(codes, "codes", false));
    FQ_TRY(check_ptr(scales, "scales", false));
    FQ_TRY(check_ptr(outer, "outer", false, 4));
    const size_t need = quant_ws(f);
    if (need > kStaticScratchBytes)
        return fail(FQ_ERR_WORKSPACE, "needs %zu bytes of scratch, the static array holds %zu",
                    need, kStaticScratchBytes);
    void *ws = nullptr;
    if (need) FQ_TRY(device_scratch(&ws));
    return run_quant(f, desc, x_bf16, rows, cols, y_bf16, codes, scales, outer, ws,
                     (hipStream_t)stream);
}

fq_status fq_fake_quant_mask(const fq_desc *desc, const void *x_bf16, int64_t rows,
                             int64_t cols, void *y_bf16, void *codes, void *scales,
                             float *outer, void *keep, void *ws, size_t ws_bytes, void *stream)
{
    Fmt f;
    FQ_TRY(check_desc(desc, &f, "desc"));
    FQ_TRY(check_shape(f, desc->axis, rows, cols));
    if (cols % 8 != 0)
        return fail(FQ_ERR_SHAPE, "cols=%lld must be a multiple of 8 for the keep mask",
                    (long long)cols);
    FQ_TRY(check_ptr(x_bf16, "x", true));
    FQ_TRY(check_ptr(y_bf16, "y", true));
    FQ_TRY(check_ptr(codes, "codes", false));
    FQ_TRY(check_ptr(scales, "scales", false));
    FQ_TRY(check_ptr(outer, "outer", false, 4));
    FQ_TRY(check_ptr(keep, "keep", true));
    const size_t need = quant_ws(f);
    if (need) {
        FQ_TRY(check_ptr(ws, "ws", true));
        if (ws_bytes < need)
            return fail(FQ_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, need);
    }
    return run_quant(f, desc, x_bf16, rows, cols, y_bf16, codes, scales, outer, ws,
                     (hipStream_t)stream, false, keep);
}

fq_status fq_fake_quant_rht(const fq_desc *desc, const void *x_bf16, int64_t rows, int64_t cols,
                            int32_t rht_block, uint64_t rht_seed, void *y_bf16, void *codes,
                            void *scales, float *outer, void *stream)
{
    Fmt f;
    FQ_TRY(check_desc(desc, &f, "desc"));
    if (f.fmt == fqimpl::FMT_NVT)
        return fail(FQ_ERR_DESC, "the rotated quantizer takes MXFP4 or NVFP4 FQ_OUTER_BLOCK128");
    if (rht_block != 16 && rht_block != 128)
        return fail(FQ_ERR_DESC, "rht_block=%d is not 16 or 128", rht_block);
    FQ_TRY(check_shape(f, desc->axis, rows, cols));
    const int64_t q = desc->axis == FQ_AXIS_ROW ? cols : rows;
    if (q % rht_block != 0)
        return fail(FQ_ERR_SHAPE, "%s=%lld must be a multiple of rht_block=%d",
                    desc->axis == FQ_AXIS_ROW ? "cols" : "rows", (long long)q, rht_block);
    FQ_TRY(check_ptr(x_bf16, "x", true));
    FQ_TRY(check_ptr(y_bf16, "y", true));
    FQ_TRY(check_ptr(codes, "codes", false));
    FQ_TRY(check_ptr(scales, "scales", false));
    FQ_TRY(check_ptr(outer, "outer", false, 4));
    return run_quant(f, desc, x_bf16, rows, cols, y_bf16, codes, scales, outer, nullptr,
                     (hipStream_t)stream, false, nullptr, rht_block, rht_seed);
}

fq_status fq_ste_backward_mask(const void *keep, const void *dy_bf16, int64_t rows,
                               int64_t cols, void *dx_bf16, void *stream)
{
    if (rows < 1 || cols < 8 || cols % 8 != 0)
        return fail(FQ_ERR_SHAPE, "rows=%lld must be >= 1 and cols=%lld a positive multiple of 8",
                    (long long)rows, (long long)cols);
    if (rows > kMaxDim || cols > kMaxDim || rows * cols > kMaxElems)
        return fail(FQ_ERR_SHAPE, "rows=%lld cols=%lld: each must be below 2^31 and rows*cols at most 2^34", (long long)rows,
                    (long long)cols);
    FQ_TRY(check_ptr(keep, "keep", true));
    FQ_TRY(check_ptr(dy_bf16, "dy", true));
    FQ_TRY(check_ptr(dx_bf16, "dx", true));
    return device_status(fqimpl::launch_ste_mask(keep, dy_bf16, rows, cols, dx_bf16,
                                                 (hipStream_t)stream),
                         "ste mask launch");
}

fq_status fq_ste_backward(const fq_desc *desc, const void *x_bf16, const void *scales,
                          const float *outer, const void *dy_bf16, int64_t rows,
                          int64_t cols, void *dx_bf16, void *stream)
{
    Fmt f;
    FQ_TRY(check_desc(desc, &f, "desc"));
    FQ_TRY(check_shape(f, desc->axis, rows, cols));
    FQ_TRY(check_ptr(x_bf16, "x", true));
    FQ_TRY(check_ptr(scales, "scales", true));
    if (f.fmt != fqimpl::FMT_MX) FQ_TRY(check_ptr(outer, "outer", true, 4));
    FQ_TRY(check_ptr(dy_bf16, "dy", true));
    FQ_TRY(check_ptr(dx_bf16, "dx", true));
    return device_status(
        fqimpl::launch_ste(f.fmt, desc->axis == FQ_AXIS_COL, x_bf16, scales,
                           f.fmt == fqimpl::FMT_MX ? nullptr : outer, dy_bf16, rows, cols,
                           dx_bf16, (hipStream_t)stream),
        "ste launch");
}

// qlinear workspace: X_hat [M, K], W_hat^T [N, K] (BF16), reduction scratch.
static size_t round256(size_t v) { return (v + 255) & ~size_t(255); }

// The MXFP4 x MXFP4 linear keeps codes and scales instead of BF16 operands,
// inside the same workspace: X codes [M, K/2], X scales [M, K/32], W codes
// and scales in the transposed layout [N, K/2], [N, K/32].
struct MxLinLayout {
    size_t xc, xs, wc, wsc;
};
static MxLinLayout mx_lin_layout(int64_t M, int64_t K, int64_t N)
{
    MxLinLayout L;
    L.xc = 0;
    L.xs = round256((size_t)M * K / 2);
    L.wc = L.xs + round256((size_t)M * K / 32);
    L.wsc = L.wc + round256((size_t)N * K / 2);
    return L;
}

size_t fq_qlinear_workspace_size(const fq_desc *desc_x, const fq_desc *desc_w, int64_t M,
                                 int64_t K, int64_t N)
{
    (void)desc_x;
    (void)desc_w;
    if (M < 1 || K < 1 || N < 1 || M > kMaxDim || K > kMaxDim || N > kMaxDim) return 0;
    if (M * K > kMaxElems || K * N > kMaxElems) return 0;
    return round256((size_t)M * K * 2) + round256((size_t)N * K * 2) +
           2 * fqimpl::kAbsmaxPartials * sizeof(uint32_t);
}

// Retained-channel fake quantization along either axis (shared by
// fq_fake_quant_retain and the linear's retained paths): the per-tensor
// format's maximum pass leaves the retained columns out.
static fq_status run_quant_retain(const Fmt &f, const fq_desc *d, uint64_t seed, const void *x,
                                  int64_t R, int64_t C, void *y, void *yt, void *codes,
                                  void *scales, float *outer, void *keep, const void *retain,
                                  const float *chan_scale, uint32_t *parts, hipStream_t st,
                                  bool cached)
{
    uint32_t npart = 0;
    if (f.fmt == fqimpl::FMT_NVT) {
        hipError_t e = fqimpl::launch_absmax(x, R * C, parts, &npart, st, retain, C);
        if (e != hipSuccess) return device_status(e, "masked tensor absmax launch");
    }
    if (d->axis == FQ_AXIS_ROW) {
        fqimpl::RetainArgs a;
        a.fmt = f.fmt;
        a.sr = d->rounding == FQ_ROUND_SR;
        a.seed = seed;
        a.x = x;
        a.R = R;
        a.C = C;
        a.retain = retain;
        a.chan_scale = chan_scale;
        a.y = y;
        a.codes = codes;
        a.scales = scales;
        a.outer = f.fmt == fqimpl::FMT_MX ? nullptr : outer;
        a.keep = keep;
        a.partials = parts;
        a.npart = npart;
        a.cached_outputs = cached;
        return device_status(fqimpl::launch_quant_retain(a, st), "retain quantize launch");
    }
    fqimpl::QuantArgs a;
    a.fmt = f.fmt;
    a.sr = d->rounding == FQ_ROUND_SR;
    a.col = 1;
    a.seed = seed;
    a.x = x;
    a.R = R;
    a.C = C;
    a.y = y;
    a.yt = yt;
    a.codes = codes;
    a.scales = scales;
    a.outer = f.fmt == fqimpl::FMT_MX ? nullptr : outer;
    a.keep = keep;
    a.partials = parts;
    a.cached_outputs = cached;
    a.retain = retain;
    a.chan_scale = chan_scale;
    return device_status(fqimpl::launch_quant(a, npart, st), "retain quantize launch");
}

// The forward; retain / chan_scale (or null) keep the activation's retained
// channels (columns of X) in FP8.
static fq_status qlinear_fwd_impl(const fq_desc *desc_x, const fq_desc *desc_w,
                                  const void *x_bf16, const void *w_bf16, int64_t M, int64_t K,
                                  int64_t N, void *y_bf16, void *ws, size_t ws_bytes,
                                  void *stream, const void *retain, const float *chan_scale)
{
    Fmt fx, fw;
    FQ_TRY(check_desc(desc_x, &fx, "desc_x"));
    FQ_TRY(check_desc(desc_w, &fw, "desc_w"));
    if (desc_x->axis != FQ_AXIS_ROW)
        return fail(FQ_ERR_DESC, "desc_x->axis must be FQ_AXIS_ROW (groups along K)");
    if (desc_w->axis != FQ_AXIS_COL)
        return fail(FQ_ERR_DESC, "desc_w->axis must be FQ_AXIS_COL (groups along K)");
    if (M < 1 || K < 1 || N < 1)
        return fail(FQ_ERR_SHAPE, "M=%lld K=%lld N=%lld must be >= 1", (long long)M,
                    (long long)K, (long long)N);
    FQ_TRY(check_shape(fx, FQ_AXIS_ROW, M, K));
    FQ_TRY(check_shape(fw, FQ_AXIS_COL, K, N));
    if (K % 64 != 0)
        return fail(FQ_ERR_SHAPE, "K=%lld must be a multiple of 64", (long long)K);
    if (M * N > kMaxElems)
        return fail(FQ_ERR_SHAPE, "M*N exceeds 2^34 elements");
    FQ_TRY(check_ptr(x_bf16, "x", true));
    FQ_TRY(check_ptr(w_bf16, "w", true));
    FQ_TRY(check_ptr(y_bf16, "y", true));
    FQ_TRY(check_ptr(ws, "ws", true));
    const size_t need = fq_qlinear_workspace_size(desc_x, desc_w, M, K, N);
    if (ws_bytes < need)
        return fail(FQ_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, need);

    char *base = (char *)ws;
    hipStream_t st = (hipStream_t)stream;
    uint32_t *parts = (uint32_t *)(base + round256((size_t)M * K * 2) + round256((size_t)N * K * 2));

    if (retain) {
        FQ_TRY(check_ptr(retain, "retain", true, 1));
        FQ_TRY(check_ptr(chan_scale, "chan_scale", true));
    }
    if (fx.fmt == fqimpl::FMT_MX && fw.fmt == fqimpl::FMT_MX && K % 64 == 0 && !retain) {
        // MXFP4 x MXFP4: the codes and E8M0 scales go straight to the scaled
        // FP4 matrix cores, nothing is dequantized
        const MxLinLayout L = mx_lin_layout(M, K, N);
        FQ_TRY(run_quant(fx, desc_x, x_bf16, M, K, nullptr, base + L.xc, base + L.xs, nullptr,
                         parts, st, /*cached=*/true));
        fqimpl::QuantArgs a;
        a.fmt = fw.fmt;
        a.sr = desc_w->rounding == FQ_ROUND_SR;
        a.col = 1;
        a.seed = desc_w->seed;
        a.x = w_bf16;
        a.R = K;
        a.C = N;
        a.y = nullptr;
        a.yt = nullptr;
        a.codes = base + L.wc;
        a.scales = base + L.wsc;
        a.outer = nullptr;
        a.partials = parts;
        a.cached_outputs = true;
        hipError_t e = fqimpl::launch_quant(a, 0, st);
        if (e != hipSuccess) return device_status(e, "transposed quantize launch");
        fqimpl::Fp4Operands o;
        o.a_codes = base + L.xc;
        o.a_scales = base + L.xs;
        o.b_codes = base + L.wc;
        o.b_scales = base + L.wsc;
        o.c = y_bf16;
        o.M = M;
        o.N = N;
        o.K = K;
        return device_status(fqimpl::launch_gemm_mxfp4_nt_pair(o, o, 1, st), "fp4 gemm launch");
    }

    void *xhat = base;
    char *what_t = base + round256((size_t)M * K * 2);
    uint32_t *parts_w = parts + fqimpl::kAbsmaxPartials;

    // both per-tensor: the two maximum passes in one launch
    int64_t npart_x = -1, npart_w = -1;
    if (fx.fmt == fqimpl::FMT_NVT && fw.fmt == fqimpl::FMT_NVT && !retain) {
        uint32_t nx = 0, nw = 0;
        hipError_t e = fqimpl::launch_absmax_pair(x_bf16, M * K, parts, &nx, w_bf16, K * N,
                                                  parts_w, &nw, st);
        if (e != hipSuccess) return device_status(e, "tensor absmax launch");
        npart_x = nx;
        npart_w = nw;
    }
    // X_hat = FQ(X) along K (rows of X), the retained channels in FP8
    if (retain)
        FQ_TRY(run_quant_retain(fx, desc_x, desc_x->seed, x_bf16, M, K, xhat, nullptr, nullptr,
                                nullptr, nullptr, nullptr, retain, chan_scale, parts, st, true));
    else
        FQ_TRY(run_quant(fx, desc_x, x_bf16, M, K, xhat, nullptr, nullptr, nullptr, parts, st,
                         /*cached=*/true, nullptr, 0, 0, npart_x));
    // W_hat^T: FQ(W) along K (columns of W), written transposed [N, K]
    {
        fqimpl::QuantArgs a;
        a.fmt = fw.fmt;
        a.sr = desc_w->rounding == FQ_ROUND_SR;
        a.col = 1;
        a.seed = desc_w->seed;
        a.x = w_bf16;
        a.R = K;
        a.C = N;
        a.y = nullptr;
        a.codes = nullptr;
        a.scales = nullptr;
        a.outer = nullptr;
        a.partials = parts_w;
        a.cached_outputs = true;
        uint32_t npart = npart_w >= 0 ? (uint32_t)npart_w : 0u;
        if (fw.fmt == fqimpl::FMT_NVT && npart_w < 0) {
            hipError_t e = fqimpl::launch_absmax(w_bf16, K * N, a.partials, &npart, st);
            if (e != hipSuccess) return device_status(e, "tensor absmax launch");
        }
        a.yt = what_t;
        hipError_t e = fqimpl::launch_quant(a, npart, st);
        if (e != hipSuccess) return device_status(e, "transposed quantize launch");
    }
    return device_status(fqimpl::launch_gemm_bf16_nt(xhat, what_t, y_bf16, M, N, K, st),
                         "gemm launch");
}

fq_status fq_qlinear_fwd(const fq_desc *desc_x, const fq_desc *desc_w, const void *x_bf16,
                         const void *w_bf16, int64_t M, int64_t K, int64_t N, void *y_bf16,
                         void *ws, size_t ws_bytes, void *stream)
{
    return qlinear_fwd_impl(desc_x, desc_w, x_bf16, w_bf16, M, K, N, y_bf16, ws, ws_bytes,
                            stream, nullptr, nullptr);
}

fq_status fq_qlinear_fwd_retain(const fq_desc *desc_x, const fq_desc *desc_w, const void *x_bf16,
                                const void *w_bf16, int64_t M, int64_t K, int64_t N,
                                const void *retain, const float *chan_scale, void *y_bf16,
                                void *ws, size_t ws_bytes, void *stream)
{
    if (!retain) return fail(FQ_ERR_NULL, "retain is NULL");
    if (!chan_scale) return fail(FQ_ERR_NULL, "chan_scale is NULL");
    if (K % 8 != 0) return fail(FQ_ERR_SHAPE, "K=%lld must be a multiple of 8", (long long)K);
    return qlinear_fwd_impl(desc_x, desc_w, x_bf16, w_bf16, M, K, N, y_bf16, ws, ws_bytes,
                            stream, retain, chan_scale);
}

// qlinear backward workspace regions, in order (each rounded up to 256 B).
struct BwdLayout {
    size_t xhat, xkeep, what, wkeep, dyq_n, wq_n, xq_mt, dyq_mt, parts, rdy_n, rw_n, rx_m, rdy_m,
        total;
};

// Backward workspace.  X_hat and W_hat are the forward's operands (BF16),
// xkeep / wkeep their STE keep masks (1 bit per element, layout of X and W);
// dyq_n, wq_n, xq_mt, dyq_mt hold the four quantized gradient-product
// operands: BF16 [M, N], [K, N], [K, M], [N, M] (transposed for the last
// two), or, for MXFP4 gradient operands, their codes followed by their E8M0
// scales in the same place (0.53 B instead of 2 B per element).
static BwdLayout bwd_layout(bool rht, int64_t M, int64_t K, int64_t N)
{
    BwdLayout L;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += round256(bytes);
        return at;
    };
    const size_t mk = (size_t)M * K, kn = (size_t)K * N, mn = (size_t)M * N;
    L.xhat = take(mk * 2);
    L.xkeep = take(mk / 8);
    L.what = take(kn * 2);
    L.wkeep = take(kn / 8);
    L.dyq_n = take(mn * 2);
    L.wq_n = take(kn * 2);
    L.xq_mt = take(mk * 2);
    L.dyq_mt = take(mn * 2);
    L.parts = take(2 * fqimpl::kAbsmaxPartials * sizeof(uint32_t));   // X, W
    // rotated operands (random Hadamard transform), only when requested
    L.rdy_n = take(rht ? mn * 2 : 0);
    L.rw_n = take(rht ? kn * 2 : 0);
    L.rx_m = take(rht ? mk * 2 : 0);
    L.rdy_m = take(rht ? mn * 2 : 0);
    L.total = off;
    return L;
}

size_t fq_qlinear_bwd_workspace_size(const fq_desc *desc_x, const fq_desc *desc_w,
                                     const fq_desc *desc_g, int32_t rht_block, int64_t M,
                                     int64_t K, int64_t N)
{
    Fmt fx, fw, fg;
    if (check_desc(desc_x, &fx, "desc_x") != FQ_OK || check_desc(desc_w, &fw, "desc_w") != FQ_OK ||
        check_desc(desc_g, &fg, "desc_g") != FQ_OK)
        return 0;
    if (rht_block != 0 && rht_block != 16 && rht_block != 128) return 0;
    if (M < 1 || K < 1 || N < 1 || M > kMaxDim || K > kMaxDim || N > kMaxDim) return 0;
    // rotated operand buffers only where the rotation cannot be fused into
    // the quantizer (per-tensor gradient format: its maximum needs a pass)
    return bwd_layout(rht_block != 0 && fg.fmt == fqimpl::FMT_NVT, M, K, N).total;
}

fq_status fq_hadamard(const void *x_bf16, int64_t rows, int64_t cols, int32_t axis,
                      int32_t block, uint64_t seed, void *y_bf16, void *stream)
{
    if (axis != FQ_AXIS_ROW && axis != FQ_AXIS_COL)
        return fail(FQ_ERR_DESC, "axis=%d is not FQ_AXIS_ROW/COL", axis);
    if (block != 16 && block != 128) return fail(FQ_ERR_DESC, "block=%d is not 16 or 128", block);
    if (rows < 1 || cols < 1) return fail(FQ_ERR_SHAPE, "rows=%lld cols=%lld must be >= 1",
                                          (long long)rows, (long long)cols);
    if (rows > kMaxDim || cols > kMaxDim || rows * cols > kMaxElems)
        return fail(FQ_ERR_SHAPE, "rows, cols must be below 2^31 and rows*cols at most 2^34");
    const int64_t q = axis == FQ_AXIS_ROW ? cols : rows;
    if (q % block != 0)
        return fail(FQ_ERR_SHAPE, "%s=%lld must be a multiple of the block %d",
                    axis == FQ_AXIS_ROW ? "cols" : "rows", (long long)q, block);
    if (axis == FQ_AXIS_COL && cols % 8 != 0)
        return fail(FQ_ERR_SHAPE, "cols=%lld must be a multiple of 8 for FQ_AXIS_COL",
                    (long long)cols);
    FQ_TRY(check_ptr(x_bf16, "x", true));
    FQ_TRY(check_ptr(y_bf16, "y", true));
    const char *xb = (const char *)x_bf16, *yb = (const char *)y_bf16;
    const size_t bytes = (size_t)rows * cols * 2;
    if (xb < yb + bytes && yb < xb + bytes) return fail(FQ_ERR_SHAPE, "x and y overlap");
    return device_status(fqimpl::launch_hadamard(x_bf16, rows, cols, axis == FQ_AXIS_COL, block,
                                                 seed, y_bf16, false, (hipStream_t)stream),
                         "hadamard launch");
}

// One quantizer pass of the backward: src [R, C] along rows (col = false,
// output y [R, C]) or along columns (col = true, output the transpose
// yt [C, R]); optional codes/scales in the pass's own layout and an optional
// keep mask in the layout of src.
static fq_status bwd_quant(const Fmt &f, const fq_desc *d, uint64_t seed, bool col,
                           const void *src, int64_t R, int64_t C, void *y, void *yt,
                           void *codes, void *scales, void *keep, uint32_t *parts,
                           hipStream_t st, int rht_n = 0, uint64_t rht_seed = 0,
                           int64_t npart_given = -1)
{
    fqimpl::QuantArgs a;
    a.fmt = f.fmt;
    a.sr = d->rounding == FQ_ROUND_SR;
    a.col = col ? 1 : 0;
    a.seed = seed;
    a.x = src;
    a.R = R;
    a.C = C;
    a.y = y;
    a.yt = yt;
    a.codes = codes;
    a.scales = scales;
    a.outer = nullptr;
    a.keep = keep;
    a.rht_n = rht_n;
    a.rht_seed = rht_seed;
    a.partials = parts;
    a.cached_outputs = true;
    // npart_given >= 0: the per-tensor partial maxima are already in parts
    uint32_t npart = npart_given >= 0 ? (uint32_t)npart_given : 0u;
    if (f.fmt == fqimpl::FMT_NVT && npart_given < 0) {
        hipError_t e = fqimpl::launch_absmax(src, R * C, parts, &npart, st);
        if (e != hipSuccess) return device_status(e, "tensor absmax launch");
    }
    return device_status(fqimpl::launch_quant(a, npart, st), "quantize launch");
}

// The backward; retain / chan_scale (or null): the activation's retained
// channels stay FP8 in X_hat and in X_hat's quantization along M, and their
// STE keep bits follow the FP8 test.
static fq_status qlinear_bwd_impl(const fq_desc *desc_x, const fq_desc *desc_w,
                                  const fq_desc *desc_g, int32_t rht_block, uint64_t rht_seed,
                                  const void *x_bf16, const void *w_bf16, const void *dy_bf16,
                                  int64_t M, int64_t K, int64_t N, void *dx_bf16, void *dw_bf16,
                                  void *ws, size_t ws_bytes, void *stream, const void *retain,
                                  const float *chan_scale)
{
    Fmt fx, fw, fg;
    FQ_TRY(check_desc(desc_x, &fx, "desc_x"));
    FQ_TRY(check_desc(desc_w, &fw, "desc_w"));
    FQ_TRY(check_desc(desc_g, &fg, "desc_g"));
    if (desc_x->axis != FQ_AXIS_ROW)
        return fail(FQ_ERR_DESC, "desc_x->axis must be FQ_AXIS_ROW (groups along K)");
    if (desc_w->axis != FQ_AXIS_COL)
        return fail(FQ_ERR_DESC, "desc_w->axis must be FQ_AXIS_COL (groups along K)");
    if (M < 1 || K < 1 || N < 1)
        return fail(FQ_ERR_SHAPE, "M=%lld K=%lld N=%lld must be >= 1", (long long)M,
                    (long long)K, (long long)N);
    // forward quantizations (X along K, W along K) and the four backward ones
    FQ_TRY(check_shape(fx, FQ_AXIS_ROW, M, K));
    FQ_TRY(check_shape(fw, FQ_AXIS_COL, K, N));
    FQ_TRY(check_shape(fg, FQ_AXIS_ROW, M, N));     // dY along N
    FQ_TRY(check_shape(fg, FQ_AXIS_ROW, K, N));     // W_hat along N
    FQ_TRY(check_shape(fg, FQ_AXIS_COL, M, K));     // X_hat along M
    FQ_TRY(check_shape(fg, FQ_AXIS_COL, M, N));     // dY along M
    if (M % 64 != 0 || N % 64 != 0)
        return fail(FQ_ERR_SHAPE, "M=%lld and N=%lld must be multiples of 64 (contractions)",
                    (long long)M, (long long)N);
    if (rht_block != 0 && rht_block != 16 && rht_block != 128)
        return fail(FQ_ERR_DESC, "rht_block=%d is not 0, 16 or 128", rht_block);
    if (rht_block != 0 && (M % rht_block != 0 || N % rht_block != 0))
        return fail(FQ_ERR_SHAPE, "M=%lld and N=%lld must be multiples of rht_block=%d",
                    (long long)M, (long long)N, rht_block);
    if (M * N > kMaxElems)
        return fail(FQ_ERR_SHAPE, "M*N exceeds 2^34 elements");
    FQ_TRY(check_ptr(x_bf16, "x", true));
    FQ_TRY(check_ptr(w_bf16, "w", true));
    FQ_TRY(check_ptr(dy_bf16, "dy", true));
    FQ_TRY(check_ptr(dx_bf16, "dx", true));
    FQ_TRY(check_ptr(dw_bf16, "dw", true));
    FQ_TRY(check_ptr(ws, "ws", true));
    const bool rht = rht_block != 0;
    // MXFP4 and double-block gradient quantizers rotate their segments in
    // registers; the per-tensor format rotates in separate passes first
    const bool rht_fused = rht && fg.fmt != fqimpl::FMT_NVT;
    const BwdLayout L = bwd_layout(rht && !rht_fused, M, K, N);
    if (ws_bytes < L.total)
        return fail(FQ_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, L.total);

    char *b = (char *)ws;
    uint32_t *parts = (uint32_t *)(b + L.parts);
    hipStream_t st = (hipStream_t)stream;
    const uint64_t sg = desc_g->seed;

    // the forward's operands and their STE keep masks: X_hat [M, K], W_hat [K, N]
    // (both per-tensor: the two maximum passes in one launch)
    uint32_t *parts_w = parts + fqimpl::kAbsmaxPartials;
    int64_t npart_x = -1, npart_w = -1;
    if (fx.fmt == fqimpl::FMT_NVT && fw.fmt == fqimpl::FMT_NVT && !retain) {
        uint32_t nx = 0, nw = 0;
        hipError_t e = fqimpl::launch_absmax_pair(x_bf16, M * K, parts, &nx, w_bf16, K * N,
                                                  parts_w, &nw, st);
        if (e != hipSuccess) return device_status(e, "tensor absmax launch");
        npart_x = nx;
        npart_w = nw;
    }
    if (retain)
        FQ_TRY(run_quant_retain(fx, desc_x, desc_x->seed, x_bf16, M, K, b + L.xhat, nullptr,
                                nullptr, nullptr, nullptr, b + L.xkeep, retain, chan_scale, parts,
                                st, true));
    else
        FQ_TRY(bwd_quant(fx, desc_x, desc_x->seed, false, x_bf16, M, K, b + L.xhat, nullptr,
                         nullptr, nullptr, b + L.xkeep, parts, st, 0, 0, npart_x));
    FQ_TRY(bwd_quant(fw, desc_w, desc_w->seed, true, w_bf16, K, N, b + L.what, nullptr,
                     nullptr, nullptr, b + L.wkeep, npart_w >= 0 ? parts_w : parts, st, 0, 0,
                     npart_w));
    // the operands before quantization, rotated along each contraction axis
    const void *op_dy_n = dy_bf16, *op_w_n = b + L.what, *op_x_m = b + L.xhat, *op_dy_m = dy_bf16;
    if (rht && !rht_fused) {
        struct { const void *src; int64_t R, C; int col; size_t dst; } rot[4] = {
            {dy_bf16, M, N, 0, L.rdy_n}, {b + L.what, K, N, 0, L.rw_n},
            {b + L.xhat, M, K, 1, L.rx_m}, {dy_bf16, M, N, 1, L.rdy_m}};
        for (const auto &r : rot) {
            hipError_t e = fqimpl::launch_hadamard(r.src, r.R, r.C, r.col, rht_block, rht_seed,
                                                   b + r.dst, true, st);
            if (e != hipSuccess) return device_status(e, "hadamard launch");
        }
        op_dy_n = b + L.rdy_n;
        op_w_n = b + L.rw_n;
        op_x_m = b + L.rx_m;
        op_dy_m = b + L.rdy_m;
    }
    // The four gradient-product operands: dY and W_hat along N (dX = Q(dY) .
    // Q(W_hat)^T), X_hat and dY along M (dW = Q(X_hat)^T . Q(dY)), Philox keys
    // seed + 0 .. 3.  Both products run in one grouped launch whose epilogue
    // applies the STE keep masks (clipped entries of dX and dW are +0).
    struct Op { const void *src; int64_t R, C; bool col; size_t at; };
    const Op ops[4] = {{op_dy_n, M, N, false, L.dyq_n}, {op_w_n, K, N, false, L.wq_n},
                       {op_x_m, M, K, true, L.xq_mt}, {op_dy_m, M, N, true, L.dyq_mt}};
    hipError_t e;
    if (fg.fmt == fqimpl::FMT_MX && !retain) {
        // MXFP4 operands go to the scaled FP4 matrix cores as codes + scales
        // (quantized along the contraction axis, which is what the product
        // needs): [rows, red/2] codes then [rows, red/32] scales
        fqimpl::Fp4Operands o[2];
        const void *cd[4], *sc[4];
        for (int i = 0; i < 4; ++i) {
            const Op &p = ops[i];
            const size_t elems = (size_t)p.R * p.C;
            void *codes = b + p.at, *scales = b + p.at + round256(elems / 2);
            FQ_TRY(bwd_quant(fg, desc_g, sg + i, p.col, p.src, p.R, p.C, nullptr, nullptr, codes,
                             scales, nullptr, parts, st, rht_fused ? rht_block : 0, rht_seed));
            cd[i] = codes;
            sc[i] = scales;
        }
        o[0] = {cd[0], sc[0], cd[1], sc[1], dx_bf16, M, K, N, b + L.xkeep};
        o[1] = {cd[2], sc[2], cd[3], sc[3], dw_bf16, K, N, M, b + L.wkeep};
        e = fqimpl::launch_gemm_mxfp4_nt_pair(o[0], o[1], 2, st);
    } else {
        // BF16 operands: row passes write y, column passes write y transposed
        // (with retained channels, X_hat along M keeps them in FP8 and the
        // products run here whatever the gradient format)
        for (int i = 0; i < 4; ++i) {
            const Op &p = ops[i];
            if (retain && i == 2) {
                fq_desc dg = *desc_g;
                dg.axis = FQ_AXIS_COL;
                FQ_TRY(run_quant_retain(fg, &dg, sg + i, p.src, p.R, p.C, nullptr, b + p.at,
                                        nullptr, nullptr, nullptr, nullptr, retain, chan_scale,
                                        parts, st, true));
                continue;
            }
            FQ_TRY(bwd_quant(fg, desc_g, sg + i, p.col, p.src, p.R, p.C, p.col ? nullptr : b + p.at,
                             p.col ? b + p.at : nullptr, nullptr, nullptr, nullptr, parts, st,
                             rht_fused ? rht_block : 0, rht_seed));
        }
        e = fqimpl::launch_gemm_bf16_nt_pair(b + L.dyq_n, b + L.wq_n, dx_bf16, M, K, N,
                                             b + L.xq_mt, b + L.dyq_mt, dw_bf16, K, N, M, st,
                                             b + L.xkeep, b + L.wkeep);
    }
    return device_status(e, "gemm launch");
}

fq_status fq_qlinear_bwd(const fq_desc *desc_x, const fq_desc *desc_w, const fq_desc *desc_g,
                         int32_t rht_block, uint64_t rht_seed, const void *x_bf16,
                         const void *w_bf16, const void *dy_bf16, int64_t M, int64_t K, int64_t N,
                         void *dx_bf16, void *dw_bf16, void *ws, size_t ws_bytes, void *stream)
{
    return qlinear_bwd_impl(desc_x, desc_w, desc_g, rht_block, rht_seed, x_bf16, w_bf16,
                            dy_bf16, M, K, N, dx_bf16, dw_bf16, ws, ws_bytes, stream, nullptr,
                            nullptr);
}

fq_status fq_qlinear_bwd_retain(const fq_desc *desc_x, const fq_desc *desc_w,
                                const fq_desc *desc_g, const void *x_bf16, const void *w_bf16,
                                const void *dy_bf16, int64_t M, int64_t K, int64_t N,
                                const void *retain, const float *chan_scale, void *dx_bf16,
                                void *dw_bf16, void *ws, size_t ws_bytes, void *stream)
{
    if (!retain) return fail(FQ_ERR_NULL, "retain is NULL");
    if (!chan_scale) return fail(FQ_ERR_NULL, "chan_scale is NULL");
    FQ_TRY(check_ptr(retain, "retain", true, 1));
    FQ_TRY(check_ptr(chan_scale, "chan_scale", true));
    if (K % 8 != 0) return fail(FQ_ERR_SHAPE, "K=%lld must be a multiple of 8", (long long)K);
    return qlinear_bwd_impl(desc_x, desc_w, desc_g, 0, 0, x_bf16, w_bf16, dy_bf16, M, K, N,
                            dx_bf16, dw_bf16, ws, ws_bytes, stream, retain, chan_scale);
}

static fq_status check_osci(const float *w, const void *q, const float *w_prev,
                            const void *q_prev, const float *dm, const float *dq, int64_t n)
{
    if (n < 4 || n % 4 != 0 || n > kMaxElems)
        return fail(FQ_ERR_SHAPE, "n=%lld must be a positive multiple of 4 up to 2^34",
                    (long long)n);
    FQ_TRY(check_ptr(w, "w", true));
    FQ_TRY(check_ptr(q, "q", true, 8));
    FQ_TRY(check_ptr(w_prev, "w_prev", true));
    FQ_TRY(check_ptr(q_prev, "q_prev", true, 8));
    FQ_TRY(check_ptr(dm, "dist_m", true));
    FQ_TRY(check_ptr(dq, "dist_q", true));
    return FQ_OK;
}

fq_status fq_osci_track(const float *w, const void *q_bf16, float *w_prev, void *q_prev_bf16,
                        float *dist_m, float *dist_q, int64_t n, int32_t first, void *stream)
{
    FQ_TRY(check_osci(w, q_bf16, w_prev, q_prev_bf16, dist_m, dist_q, n));
    return device_status(fqimpl::launch_osci_track(w, q_bf16, w_prev, q_prev_bf16, dist_m,
                                                   dist_q, n, first ? 1 : 0,
                                                   (hipStream_t)stream),
                         "osci track launch");
}

fq_status fq_osci_reset(const fq_desc *desc, float *w, const void *q_bf16, const void *codes,
                        const void *scales, const float *outer, int64_t rows, int64_t cols,
                        float *w_prev, void *q_prev_bf16, float *dist_m, float *dist_q,
                        float tau, int32_t target, void *stream)
{
    if (target != FQ_OSCI_BIN_CENTRE && target != FQ_OSCI_GRID_VALUE)
        return fail(FQ_ERR_DESC, "target=%d is not FQ_OSCI_BIN_CENTRE/GRID_VALUE", target);
    if (rows < 1 || cols < 1 || rows > kMaxDim || cols > kMaxDim ||
        rows * cols > kMaxElems)
        return fail(FQ_ERR_SHAPE, "rows=%lld cols=%lld out of range", (long long)rows,
                    (long long)cols);
    if (cols % 4 != 0)
        return fail(FQ_ERR_SHAPE, "cols=%lld must be a multiple of 4", (long long)cols);
    const int64_t n = rows * cols;
    FQ_TRY(check_osci(w, q_bf16, w_prev, q_prev_bf16, dist_m, dist_q, n));
    if (!(tau >= 0.0f) || tau > 3.4e38f)
        return fail(FQ_ERR_DESC, "tau=%g must be finite and >= 0", (double)tau);
    fqimpl::OsciResetArgs a;
    a.w = w;
    a.q = q_bf16;
    a.w_prev = w_prev;
    a.q_prev = q_prev_bf16;
    a.dist_m = dist_m;
    a.dist_q = dist_q;
    a.n = n;
    a.R = rows;
    a.C = cols;
    a.tau = tau;
    a.grid_target = target == FQ_OSCI_GRID_VALUE;
    a.fmt = fqimpl::FMT_MX;
    a.col = false;
    a.codes = a.scales = nullptr;
    a.outer = nullptr;
    if (!a.grid_target) {
        Fmt f;
        FQ_TRY(check_desc(desc, &f, "desc"));
        FQ_TRY(check_shape(f, desc->axis, rows, cols));
        FQ_TRY(check_ptr(codes, "codes", true));
        FQ_TRY(check_ptr(scales, "scales", true));
        FQ_TRY(check_ptr(outer, "outer", f.fmt != fqimpl::FMT_MX, 4));
        a.fmt = f.fmt;
        a.col = desc->axis == FQ_AXIS_COL;
        a.codes = codes;
        a.scales = scales;
        a.outer = f.fmt == fqimpl::FMT_MX ? nullptr : outer;
    }
    return device_status(fqimpl::launch_osci_reset(a, (hipStream_t)stream), "osci reset launch");
}

fq_status fq_channel_absmax(const void *x_bf16, int64_t rows, int64_t cols, uint32_t *amax,
                            void *stream)
{
    if (rows < 1 || cols < 8 || cols % 8 != 0)
        return fail(FQ_ERR_SHAPE, "rows=%lld must be >= 1 and cols=%lld a positive multiple of 8",
                    (long long)rows, (long long)cols);
    if (rows > kMaxDim || cols > kMaxDim || rows * cols > kMaxElems)
        return fail(FQ_ERR_SHAPE, "rows, cols must be below 2^31 and rows*cols at most 2^34");
    FQ_TRY(check_ptr(x_bf16, "x", true));
    FQ_TRY(check_ptr(amax, "amax", true, 4));
    return device_status(fqimpl::launch_channel_absmax(x_bf16, rows, cols, amax,
                                                       (hipStream_t)stream),
                         "channel absmax launch");
}

fq_status fq_select_channels(const uint32_t *amax, int64_t cols, int64_t k, void *retain,
                             float *chan_scale, void *stream)
{
    if (cols < 8 || cols % 8 != 0 || cols > (int64_t(1) << 24))
        return fail(FQ_ERR_SHAPE, "cols=%lld must be a positive multiple of 8 up to 2^24",
                    (long long)cols);
    if (k < 0 || k > cols)
        return fail(FQ_ERR_SHAPE, "k=%lld must be in [0, cols=%lld]", (long long)k,
                    (long long)cols);
    FQ_TRY(check_ptr(amax, "amax", true, 4));
    FQ_TRY(check_ptr(retain, "retain", true, 1));
    FQ_TRY(check_ptr(chan_scale, "chan_scale", true, 4));
    return device_status(fqimpl::launch_select_channels(amax, cols, k, retain, chan_scale,
                                                        (hipStream_t)stream),
                         "select channels launch");
}

fq_status fq_fake_quant_retain(const fq_desc *desc, const void *x_bf16, int64_t rows,
                               int64_t cols, void *y_bf16, void *codes, void *scales,
                               float *outer, const void *retain, const float *chan_scale,
                               void *ws, size_t ws_bytes, void *stream)
{
    Fmt f;
    FQ_TRY(check_desc(desc, &f, "desc"));
    FQ_TRY(check_shape(f, desc->axis, rows, cols));
    if (cols % 8 != 0)
        return fail(FQ_ERR_SHAPE, "cols=%lld must be a multiple of 8 (channel mask bytes)",
                    (long long)cols);
    FQ_TRY(check_ptr(x_bf16, "x", true));
    FQ_TRY(check_ptr(y_bf16, "y", true));
    FQ_TRY(check_ptr(codes, "codes", false));
    FQ_TRY(check_ptr(scales, "scales", false));
    FQ_TRY(check_ptr(outer, "outer", false, 4));
    FQ_TRY(check_ptr(retain, "retain", true, 1));
    FQ_TRY(check_ptr(chan_scale, "chan_scale", true));
    const size_t need = quant_ws(f);
    if (need) {
        FQ_TRY(check_ptr(ws, "ws", true));
        if (ws_bytes < need)
            return fail(FQ_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, need);
    }
    return run_quant_retain(f, desc, desc->seed, x_bf16, rows, cols, y_bf16, nullptr, codes,
                            scales, outer, nullptr, retain, chan_scale, (uint32_t *)ws,
                            (hipStream_t)stream, false);
}

const char *fq_status_string(fq_status s)
{
    switch (s) {
    case FQ_OK: return "FQ_OK";
    case FQ_ERR_NULL: return "FQ_ERR_NULL: a required pointer is NULL";
    case FQ_ERR_DESC: return "FQ_ERR_DESC: unsupported descriptor";
    case FQ_ERR_SHAPE: return "FQ_ERR_SHAPE: unsupported shape";
    case FQ_ERR_ALIGN: return "FQ_ERR_ALIGN: misaligned pointer";
    case FQ_ERR_WORKSPACE: return "FQ_ERR_WORKSPACE: workspace too small";
    case FQ_ERR_DEVICE: return "FQ_ERR_DEVICE: HIP launch failed";
    }
    return "unknown fq_status";
}

const char *fq_last_error(void) { return g_err; }

const char *fq_version(void) { return "0.1.0"; }

}  // extern "C"
