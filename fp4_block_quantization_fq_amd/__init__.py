"""Blockwise FP4 (MXFP4 / NVFP4) fake quantization on AMD MI355X (gfx950).

Thin ctypes binding over libfq.so (C ABI in include/fq.h).  Every function
here only marshals arguments: shapes, device pointers and the current HIP
stream go to the library, and all arithmetic runs in its HIP kernels.  PyTorch
supplies device memory and streams.  There is no fallback: if libfq.so is
missing or a call fails, an exception is raised.

Tensors: BF16 data is passed as torch.bfloat16 tensors; codes and scales as
torch.uint8; outer scales as torch.float32.  Layouts are those of fq.h.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfq.so")

FQ_OK, FQ_ERR_NULL, FQ_ERR_DESC, FQ_ERR_SHAPE, FQ_ERR_ALIGN, FQ_ERR_WORKSPACE, FQ_ERR_DEVICE = range(7)
FQ_SCALE_E8M0, FQ_SCALE_E4M3 = 0, 1
FQ_OUTER_NONE, FQ_OUTER_TENSOR, FQ_OUTER_BLOCK128 = 0, 1, 2
FQ_ROUND_RNE, FQ_ROUND_SR = 0, 1
FQ_AXIS_ROW, FQ_AXIS_COL = 0, 1
FQ_OSCI_BIN_CENTRE, FQ_OSCI_GRID_VALUE = 0, 1

# every symbol include/fq.h declares
EXPORTED = (
    "fq_desc_mxfp4", "fq_desc_nvfp4", "fq_workspace_size", "fq_quantize",
    "fq_dequantize", "fq_fake_quant", "fq_fake_quant_mask", "fq_ste_backward",
    "fq_ste_backward_mask", "fq_osci_track", "fq_osci_reset", "fq_channel_absmax",
    "fq_select_channels", "fq_fake_quant_retain", "fq_fake_quant_rht",
    "fq_qlinear_workspace_size", "fq_qlinear_fwd", "fq_hadamard",
    "fq_qlinear_bwd_workspace_size", "fq_qlinear_bwd", "fq_status_string",
    "fq_last_error", "fq_version", "fq_fake_quant_noalloc", "fq_qlinear_fwd_retain",
    "fq_qlinear_bwd_retain",
)


class FqDesc(ctypes.Structure):
    _fields_ = [
        ("block_size", ctypes.c_int32),
        ("scale_type", ctypes.c_int32),
        ("outer", ctypes.c_int32),
        ("rounding", ctypes.c_int32),
        ("axis", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("seed", ctypes.c_uint64),
    ]

    def __repr__(self):
        return (f"FqDesc(block_size={self.block_size}, scale_type={self.scale_type}, "
                f"outer={self.outer}, rounding={self.rounding}, axis={self.axis}, "
                f"seed={self.seed})")


class FqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libfq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m fp4_block_quantization_fq_amd.build` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        dp = ctypes.POINTER(FqDesc)
        L.fq_desc_mxfp4.argtypes = []
        L.fq_desc_mxfp4.restype = FqDesc
        L.fq_desc_nvfp4.argtypes = []
        L.fq_desc_nvfp4.restype = FqDesc
        L.fq_workspace_size.argtypes = [dp, i64, i64]
        L.fq_workspace_size.restype = sz
        L.fq_quantize.argtypes = [dp, vp, i64, i64, vp, vp, vp, vp, sz, vp]
        L.fq_quantize.restype = ctypes.c_int
        L.fq_dequantize.argtypes = [dp, vp, vp, vp, i64, i64, vp, vp]
        L.fq_dequantize.restype = ctypes.c_int
        L.fq_fake_quant.argtypes = [dp, vp, i64, i64, vp, vp, vp, vp, vp, sz, vp]
        L.fq_fake_quant.restype = ctypes.c_int
        L.fq_fake_quant_noalloc.argtypes = [dp, vp, i64, i64, vp, vp, vp, vp, vp]
        L.fq_fake_quant_noalloc.restype = ctypes.c_int
        L.fq_ste_backward.argtypes = [dp, vp, vp, vp, vp, i64, i64, vp, vp]
        L.fq_fake_quant_mask.restype = ctypes.c_int
        L.fq_fake_quant_mask.argtypes = [dp, vp, i64, i64, vp, vp, vp, vp, vp, vp, sz, vp]
        L.fq_ste_backward_mask.restype = ctypes.c_int
        f32 = ctypes.c_float
        L.fq_osci_track.argtypes = [vp, vp, vp, vp, vp, vp, i64, ctypes.c_int32, vp]
        L.fq_osci_track.restype = ctypes.c_int
        L.fq_osci_reset.argtypes = [ctypes.POINTER(FqDesc), vp, vp, vp, vp, vp, i64, i64, vp, vp,
                                    vp, vp, f32, ctypes.c_int32, vp]
        L.fq_osci_reset.restype = ctypes.c_int
        L.fq_channel_absmax.argtypes = [vp, i64, i64, vp, vp]
        L.fq_channel_absmax.restype = ctypes.c_int
        L.fq_select_channels.argtypes = [vp, i64, i64, vp, vp, vp]
        L.fq_select_channels.restype = ctypes.c_int
        L.fq_fake_quant_retain.argtypes = [dp, vp, i64, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.fq_fake_quant_retain.restype = ctypes.c_int
        L.fq_fake_quant_rht.argtypes = [dp, vp, i64, i64, ctypes.c_int32, ctypes.c_uint64, vp, vp,
                                        vp, vp, vp]
        L.fq_fake_quant_rht.restype = ctypes.c_int
        L.fq_ste_backward_mask.argtypes = [vp, vp, i64, i64, vp, vp]
        L.fq_ste_backward.restype = ctypes.c_int
        L.fq_qlinear_workspace_size.argtypes = [dp, dp, i64, i64, i64]
        L.fq_qlinear_workspace_size.restype = sz
        L.fq_qlinear_fwd.argtypes = [dp, dp, vp, vp, i64, i64, i64, vp, vp, sz, vp]
        L.fq_qlinear_fwd.restype = ctypes.c_int
        i32, u64 = ctypes.c_int32, ctypes.c_uint64
        L.fq_hadamard.argtypes = [vp, i64, i64, i32, i32, u64, vp, vp]
        L.fq_hadamard.restype = ctypes.c_int
        L.fq_qlinear_bwd_workspace_size.argtypes = [dp, dp, dp, i32, i64, i64, i64]
        L.fq_qlinear_bwd_workspace_size.restype = sz
        L.fq_qlinear_bwd.argtypes = [dp, dp, dp, i32, u64, vp, vp, vp, i64, i64, i64, vp, vp, vp,
                                     sz, vp]
        L.fq_qlinear_bwd.restype = ctypes.c_int
        L.fq_qlinear_fwd_retain.argtypes = [dp, dp, vp, vp, i64, i64, i64, vp, vp, vp, vp, sz,
                                            vp]
        L.fq_qlinear_fwd_retain.restype = ctypes.c_int
        L.fq_qlinear_bwd_retain.argtypes = [dp, dp, dp, vp, vp, vp, i64, i64, i64, vp, vp, vp, vp,
                                            vp, sz, vp]
        L.fq_qlinear_bwd_retain.restype = ctypes.c_int
        L.fq_status_string.argtypes = [ctypes.c_int]
        L.fq_status_string.restype = ctypes.c_char_p
        L.fq_last_error.argtypes = []
        L.fq_last_error.restype = ctypes.c_char_p
        L.fq_version.argtypes = []
        L.fq_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int):
    if status != FQ_OK:
        msg = lib().fq_last_error().decode() or lib().fq_status_string(status).decode()
        raise FqError(status, msg)


# ---------------------------------------------------------------------------
# descriptors
# ---------------------------------------------------------------------------

def fq_desc_mxfp4(rounding: int = FQ_ROUND_RNE, axis: int = FQ_AXIS_ROW, seed: int = 0) -> FqDesc:
    d = lib().fq_desc_mxfp4()
    d.rounding, d.axis, d.seed = rounding, axis, seed
    return d


def fq_desc_nvfp4(rounding: int = FQ_ROUND_RNE, axis: int = FQ_AXIS_ROW, seed: int = 0,
                  outer: int = FQ_OUTER_TENSOR) -> FqDesc:
    d = lib().fq_desc_nvfp4()
    d.rounding, d.axis, d.seed, d.outer = rounding, axis, seed, outer
    return d


def block_size(desc: FqDesc) -> int:
    return desc.block_size


# ---------------------------------------------------------------------------
# tensor plumbing
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t, nbytes: int | None = None, name: str = "buffer", elem: int | None = None):
    """Device pointer of a tensor the library will read or write.  The C
    library sees only pointers and sizes, so the binding checks here what it
    cannot: the tensor is on the GPU, contiguous, of the expected element
    size, and holds at least `nbytes` bytes (a smaller buffer would be written
    past its end)."""
    if t is None:
        return None
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")
    if elem is not None and t.element_size() != elem:
        raise ValueError(f"{name} has {t.element_size()}-byte elements, expected {elem}")
    if nbytes is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, "
                         f"{nbytes} are needed")
    return ctypes.c_void_p(t.data_ptr())


def _bf16(t, rows: int, cols: int, name: str):
    """A BF16 [rows, cols] operand (2-byte elements)."""
    return _ptr(t, rows * cols * 2, name, elem=2)


def _qptrs(desc, out, rows: int, cols: int):
    """Pointers of the codes, scales and outer outputs, checked against the
    sizes the descriptor implies (each may be None)."""
    if out is None:
        return None, None, None
    s = output_shapes(desc, rows, cols)
    n = lambda shp: 0 if shp is None else math.prod(shp)
    return (_ptr(out.codes, n(s["codes"]), "codes"), _ptr(out.scales, n(s["scales"]), "scales"),
            _ptr(out.outer, 4 * n(s["outer"]), "outer"))


def _stream(stream=None):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


@dataclass
class Quantized:
    codes: "object"
    scales: "object"
    outer: "object"


def output_shapes(desc: FqDesc, rows: int, cols: int) -> dict:
    """Shapes of codes, scales and outer for x of shape [rows, cols]."""
    qr, qc = (rows, cols) if desc.axis == FQ_AXIS_ROW else (cols, rows)
    B = desc.block_size
    shapes = {"codes": (qr, qc // 2), "scales": (qr, qc // B)}
    if desc.outer == FQ_OUTER_TENSOR:
        shapes["outer"] = (1,)
    elif desc.outer == FQ_OUTER_BLOCK128:
        shapes["outer"] = (qr, qc // 128)
    else:
        shapes["outer"] = None
    return shapes


def alloc_outputs(desc: FqDesc, rows: int, cols: int, device) -> Quantized:
    torch = _torch()
    s = output_shapes(desc, rows, cols)
    codes = torch.empty(s["codes"], dtype=torch.uint8, device=device)
    scales = torch.empty(s["scales"], dtype=torch.uint8, device=device)
    outer = None if s["outer"] is None else torch.empty(s["outer"], dtype=torch.float32, device=device)
    return Quantized(codes, scales, outer)


def workspace(desc: FqDesc, rows: int, cols: int, device):
    torch = _torch()
    n = lib().fq_workspace_size(ctypes.byref(desc), rows, cols)
    return torch.empty((max(n, 16),), dtype=torch.uint8, device=device), n


# ---------------------------------------------------------------------------
# the five operations
# ---------------------------------------------------------------------------

def fq_quantize(desc: FqDesc, x, out: Quantized | None = None, ws=None, stream=None) -> Quantized:
    rows, cols = x.shape
    if out is None:
        out = alloc_outputs(desc, rows, cols, x.device)
    if ws is None:
        ws, nbytes = workspace(desc, rows, cols, x.device)
    else:
        nbytes = ws.numel() * ws.element_size()
    codes, scales, outer = _qptrs(desc, out, rows, cols)
    _check(lib().fq_quantize(ctypes.byref(desc), _bf16(x, rows, cols, "x"), rows, cols, codes,
                             scales, outer, _ptr(ws, nbytes, "ws"), nbytes, _stream(stream)))
    return out


def fq_dequantize(desc: FqDesc, q: Quantized, rows: int, cols: int, y=None, stream=None):
    torch = _torch()
    if y is None:
        y = torch.empty((rows, cols), dtype=torch.bfloat16, device=q.codes.device)
    codes, scales, outer = _qptrs(desc, q, rows, cols)
    _check(lib().fq_dequantize(ctypes.byref(desc), codes, scales, outer, rows, cols,
                               _bf16(y, rows, cols, "y"), _stream(stream)))
    return y


def fq_fake_quant(desc: FqDesc, x, y=None, out: Quantized | None = None, ws=None,
                  stream=None):
    """y = dequantize(quantize(x)); also fills `out` (codes, scales, outer) if
    given.  Returns y."""
    torch = _torch()
    rows, cols = x.shape
    if y is None:
        y = torch.empty_like(x)
    if ws is None:
        ws, nbytes = workspace(desc, rows, cols, x.device)
    else:
        nbytes = ws.numel() * ws.element_size()
    codes, scales, outer = _qptrs(desc, out, rows, cols)
    _check(lib().fq_fake_quant(ctypes.byref(desc), _bf16(x, rows, cols, "x"), rows, cols,
                               _bf16(y, rows, cols, "y"), codes, scales, outer,
                               _ptr(ws, nbytes, "ws"), nbytes, _stream(stream)))
    return y


def fq_fake_quant_noalloc(desc: FqDesc, x, y, out: Quantized | None = None, stream=None):
    """fq_fake_quant with the library's own per-GPU scratch instead of a
    workspace (the C call allocates nothing; y and out are the caller's).
    Returns y."""
    rows, cols = x.shape
    codes, scales, outer = _qptrs(desc, out, rows, cols)
    _check(lib().fq_fake_quant_noalloc(ctypes.byref(desc), _bf16(x, rows, cols, "x"), rows, cols,
                                       _bf16(y, rows, cols, "y"), codes, scales, outer,
                                       _stream(stream)))
    return y


def fq_fake_quant_mask(desc: FqDesc, x, y=None, out: Quantized | None = None, keep=None,
                       ws=None, stream=None):
    """fq_fake_quant that also writes the STE keep mask (uint8 [rows, cols/8],
    layout of x, bit c mod 8 of byte (r, c/8) set where element (r, c) was
    kept).  Returns (y, keep)."""
    torch = _torch()
    rows, cols = x.shape
    if y is None:
        y = torch.empty_like(x)
    if keep is None:
        keep = torch.empty((rows, cols // 8), dtype=torch.uint8, device=x.device)
    if ws is None:
        ws, nbytes = workspace(desc, rows, cols, x.device)
    else:
        nbytes = ws.numel() * ws.element_size()
    codes, scales, outer = _qptrs(desc, out, rows, cols)
    _check(lib().fq_fake_quant_mask(ctypes.byref(desc), _bf16(x, rows, cols, "x"), rows, cols,
                                    _bf16(y, rows, cols, "y"), codes, scales, outer,
                                    _ptr(keep, rows * cols // 8, "keep"),
                                    _ptr(ws, nbytes, "ws"), nbytes, _stream(stream)))
    return y, keep


def fq_ste_backward_mask(keep, dy, dx=None, stream=None):
    """dx = dy where the keep bit is set, else +0.  Returns dx."""
    torch = _torch()
    rows, cols = dy.shape
    if dx is None:
        dx = torch.empty_like(dy)
    _check(lib().fq_ste_backward_mask(_ptr(keep, rows * cols // 8, "keep"),
                                      _bf16(dy, rows, cols, "dy"), rows, cols,
                                      _bf16(dx, rows, cols, "dx"), _stream(stream)))
    return dx


def osci_state(n: int, device):
    """OsciReset state for n weights: w_prev, dist_m, dist_q FP32 and q_prev BF16."""
    torch = _torch()
    return {"w_prev": torch.zeros(n, dtype=torch.float32, device=device),
            "q_prev": torch.zeros(n, dtype=torch.bfloat16, device=device),
            "dist_m": torch.zeros(n, dtype=torch.float32, device=device),
            "dist_q": torch.zeros(n, dtype=torch.float32, device=device)}


def _osci_ptrs(w, q, st: dict, n: int):
    return (_ptr(w, 4 * n, "w", elem=4), _ptr(q, 2 * n, "q", elem=2),
            _ptr(st["w_prev"], 4 * n, "w_prev", elem=4), _ptr(st["q_prev"], 2 * n, "q_prev", elem=2),
            _ptr(st["dist_m"], 4 * n, "dist_m", elem=4), _ptr(st["dist_q"], 4 * n, "dist_q", elem=4))


def fq_osci_track(w, q, st: dict, first: bool = False, stream=None):
    """One step of the oscillation tracker (w FP32 master, q BF16 quantized)."""
    n = w.numel()
    _check(lib().fq_osci_track(*_osci_ptrs(w, q, st, n), n, 1 if first else 0, _stream(stream)))


def fq_osci_reset(w, q, st: dict, tau: float, desc=None, quant=None,
                  target: int = FQ_OSCI_BIN_CENTRE, stream=None):
    """The OsciReset check: oscillating master weights (in place in w, an FP32
    [rows, cols] tensor) go to the centre of their current quantization bin,
    read from `quant` (the Quantized outputs of the quantization with `desc`
    that gave q), or with target=FQ_OSCI_GRID_VALUE to q itself; every
    element starts a new window."""
    assert w.dim() == 2, "w must be [rows, cols]"
    rows, cols = w.shape
    n = rows * cols
    ptrs = _osci_ptrs(w, q, st, n)
    if target == FQ_OSCI_GRID_VALUE:
        d, codes, scales, outer = None, None, None, None
    else:
        d = ctypes.byref(desc)
        codes, scales, outer = _qptrs(desc, quant, rows, cols)
    _check(lib().fq_osci_reset(d, ptrs[0], ptrs[1], codes, scales, outer, rows, cols, *ptrs[2:],
                               ctypes.c_float(tau), target, _stream(stream)))


def fq_channel_absmax(x, amax=None, stream=None):
    """Fold max |x[:, c]| (BF16 magnitude bits) into amax [cols] (int32
    tensor, zeros if not given).  Returns amax."""
    torch = _torch()
    rows, cols = x.shape
    if amax is None:
        amax = torch.zeros(cols, dtype=torch.int32, device=x.device)
    _check(lib().fq_channel_absmax(_bf16(x, rows, cols, "x"), rows, cols,
                                   _ptr(amax, 4 * cols, "amax", elem=4), _stream(stream)))
    return amax


def fq_select_channels(amax, k: int, stream=None):
    """The k largest channels: (retain uint8 [cols/8] bit mask, chan_scale
    float32 [cols])."""
    torch = _torch()
    cols = amax.numel()
    retain = torch.empty(cols // 8, dtype=torch.uint8, device=amax.device)
    scale = torch.empty(cols, dtype=torch.float32, device=amax.device)
    _check(lib().fq_select_channels(_ptr(amax, 4 * cols, "amax", elem=4), cols, k,
                                    _ptr(retain), _ptr(scale), _stream(stream)))
    return retain, scale


def fq_fake_quant_retain(desc: FqDesc, x, retain, chan_scale, y=None,
                         out: Quantized | None = None, ws=None, stream=None):
    """Fake quantization (either axis, any format) with the retained channels
    (columns of x) in FP8.  Returns y."""
    torch = _torch()
    rows, cols = x.shape
    if y is None:
        y = torch.empty_like(x)
    if ws is None:
        ws, nbytes = workspace(desc, rows, cols, x.device)
    else:
        nbytes = ws.numel() * ws.element_size()
    codes, scales, outer = _qptrs(desc, out, rows, cols)
    _check(lib().fq_fake_quant_retain(ctypes.byref(desc), _bf16(x, rows, cols, "x"), rows, cols,
                                      _bf16(y, rows, cols, "y"), codes, scales, outer,
                                      _ptr(retain, cols // 8, "retain"),
                                      _ptr(chan_scale, 4 * cols, "chan_scale", elem=4),
                                      _ptr(ws, nbytes, "ws"), nbytes, _stream(stream)))
    return y


def fq_fake_quant_rht(desc: FqDesc, x, rht_block: int, rht_seed: int, y=None,
                      out: Quantized | None = None, stream=None):
    """Fake quantization of the random Hadamard rotation of x along the
    quantization axis, in one pass.  Returns y."""
    torch = _torch()
    rows, cols = x.shape
    if y is None:
        y = torch.empty_like(x)
    codes, scales, outer = _qptrs(desc, out, rows, cols)
    _check(lib().fq_fake_quant_rht(ctypes.byref(desc), _bf16(x, rows, cols, "x"), rows, cols,
                                   rht_block, rht_seed, _bf16(y, rows, cols, "y"), codes, scales,
                                   outer, _stream(stream)))
    return y


def fq_ste_backward(desc: FqDesc, x, q: Quantized, dy, dx=None, stream=None):
    torch = _torch()
    rows, cols = x.shape
    if dx is None:
        dx = torch.empty_like(dy)
    _, scales, outer = _qptrs(desc, Quantized(None, q.scales, q.outer), rows, cols)
    _check(lib().fq_ste_backward(ctypes.byref(desc), _bf16(x, rows, cols, "x"), scales, outer,
                                 _bf16(dy, rows, cols, "dy"), rows, cols,
                                 _bf16(dx, rows, cols, "dx"), _stream(stream)))
    return dx


def qlinear_workspace(desc_x: FqDesc, desc_w: FqDesc, M: int, K: int, N: int, device):
    torch = _torch()
    n = lib().fq_qlinear_workspace_size(ctypes.byref(desc_x), ctypes.byref(desc_w), M, K, N)
    return torch.empty((n,), dtype=torch.uint8, device=device)


def qlinear_workspace_views(ws, M: int, K: int, N: int):
    """(X_hat [M, K], W_hat^T [N, K]) views into a qlinear workspace."""
    torch = _torch()
    off = (M * K * 2 + 255) // 256 * 256
    xhat = ws[: M * K * 2].view(torch.bfloat16).view(M, K)
    what_t = ws[off: off + N * K * 2].view(torch.bfloat16).view(N, K)
    return xhat, what_t


def qlinear_workspace_mx_views(ws, M: int, K: int, N: int):
    """(X codes [M, K/2], X scales [M, K/32], W^T codes [N, K/2], W^T scales
    [N, K/32]) in a qlinear workspace used by an MXFP4 x MXFP4 linear."""
    r = lambda v: (v + 255) // 256 * 256
    c1 = r(M * K // 2)
    c2 = c1 + r(M * K // 32)
    c3 = c2 + r(N * K // 2)
    return (ws[: M * K // 2].view(M, K // 2), ws[c1: c1 + M * K // 32].view(M, K // 32),
            ws[c2: c2 + N * K // 2].view(N, K // 2), ws[c3: c3 + N * K // 32].view(N, K // 32))


def fq_qlinear_fwd(desc_x: FqDesc, desc_w: FqDesc, x, w, y=None, ws=None, stream=None):
    """Y [M, N] = FQ(X) @ FQ(W) (BF16 out, FP32 accumulation)."""
    torch = _torch()
    M, K = x.shape
    K2, N = w.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {x.shape} @ {w.shape}")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = qlinear_workspace(desc_x, desc_w, M, K, N, x.device)
    _check(lib().fq_qlinear_fwd(ctypes.byref(desc_x), ctypes.byref(desc_w), _bf16(x, M, K, "x"),
                                _bf16(w, K, N, "w"), M, K, N, _bf16(y, M, N, "y"),
                                _ptr(ws, None, "ws", elem=1), ws.numel(), _stream(stream)))
    return y


def fq_hadamard(x, block: int, axis: int = FQ_AXIS_ROW, seed: int = 0, y=None, stream=None):
    """Random Hadamard transform of a [R, C] BF16 tensor in blocks of 16 or 128."""
    torch = _torch()
    rows, cols = x.shape
    if y is None:
        y = torch.empty_like(x)
    _check(lib().fq_hadamard(_bf16(x, rows, cols, "x"), rows, cols, axis, block, seed,
                             _bf16(y, rows, cols, "y"), _stream(stream)))
    return y


def qlinear_bwd_workspace(desc_x: FqDesc, desc_w: FqDesc, desc_g: FqDesc, M: int, K: int,
                          N: int, device, rht_block: int = 0):
    torch = _torch()
    n = lib().fq_qlinear_bwd_workspace_size(ctypes.byref(desc_x), ctypes.byref(desc_w),
                                            ctypes.byref(desc_g), rht_block, M, K, N)
    return torch.empty((n,), dtype=torch.uint8, device=device)


def fq_qlinear_bwd(desc_x: FqDesc, desc_w: FqDesc, desc_g: FqDesc, x, w, dy, dx=None, dw=None,
                   ws=None, stream=None, rht_block: int = 0, rht_seed: int = 0):
    """(dX [M, K], dW [K, N]) of Y = FQ(X) @ FQ(W) for the upstream gradient dY [M, N];
    rht_block 16/128 rotates each product's operands by the random Hadamard transform."""
    torch = _torch()
    M, K = x.shape
    K2, N = w.shape
    if K2 != K or tuple(dy.shape) != (M, N):
        raise ValueError(f"shapes differ: x {tuple(x.shape)}, w {tuple(w.shape)}, dy {tuple(dy.shape)}")
    if dx is None:
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=x.device)
    if dw is None:
        dw = torch.empty((K, N), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = qlinear_bwd_workspace(desc_x, desc_w, desc_g, M, K, N, x.device, rht_block)
    _check(lib().fq_qlinear_bwd(ctypes.byref(desc_x), ctypes.byref(desc_w), ctypes.byref(desc_g),
                                rht_block, rht_seed, _bf16(x, M, K, "x"), _bf16(w, K, N, "w"),
                                _bf16(dy, M, N, "dy"), M, K, N, _bf16(dx, M, K, "dx"),
                                _bf16(dw, K, N, "dw"), _ptr(ws, None, "ws", elem=1), ws.numel(),
                                _stream(stream)))
    return dx, dw


def fq_qlinear_fwd_retain(desc_x: FqDesc, desc_w: FqDesc, x, w, retain, chan_scale, y=None,
                          ws=None, stream=None):
    """Y = FQ(X) @ FQ(W) with X's retained channels (retain [K/8], chan_scale
    [K]) in FP8."""
    torch = _torch()
    M, K = x.shape
    K2, N = w.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {x.shape} @ {w.shape}")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = qlinear_workspace(desc_x, desc_w, M, K, N, x.device)
    _check(lib().fq_qlinear_fwd_retain(ctypes.byref(desc_x), ctypes.byref(desc_w),
                                       _bf16(x, M, K, "x"), _bf16(w, K, N, "w"), M, K, N,
                                       _ptr(retain, K // 8, "retain"),
                                       _ptr(chan_scale, 4 * K, "chan_scale", elem=4),
                                       _bf16(y, M, N, "y"), _ptr(ws, None, "ws", elem=1),
                                       ws.numel(), _stream(stream)))
    return y


def fq_qlinear_bwd_retain(desc_x: FqDesc, desc_w: FqDesc, desc_g: FqDesc, x, w, dy, retain,
                          chan_scale, dx=None, dw=None, ws=None, stream=None):
    """(dX, dW) of the linear with X's retained channels in FP8 in the forward
    and the backward."""
    torch = _torch()
    M, K = x.shape
    K2, N = w.shape
    if K2 != K or tuple(dy.shape) != (M, N):
        raise ValueError(f"shapes differ: x {tuple(x.shape)}, w {tuple(w.shape)}, dy {tuple(dy.shape)}")
    if dx is None:
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=x.device)
    if dw is None:
        dw = torch.empty((K, N), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = qlinear_bwd_workspace(desc_x, desc_w, desc_g, M, K, N, x.device, 0)
    _check(lib().fq_qlinear_bwd_retain(ctypes.byref(desc_x), ctypes.byref(desc_w),
                                       ctypes.byref(desc_g), _bf16(x, M, K, "x"),
                                       _bf16(w, K, N, "w"), _bf16(dy, M, N, "dy"), M, K, N,
                                       _ptr(retain, K // 8, "retain"),
                                       _ptr(chan_scale, 4 * K, "chan_scale", elem=4),
                                       _bf16(dx, M, K, "dx"), _bf16(dw, K, N, "dw"),
                                       _ptr(ws, None, "ws", elem=1), ws.numel(), _stream(stream)))
    return dx, dw


def version() -> str:
    return lib().fq_version().decode()
