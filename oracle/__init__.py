"""CPU oracle for blockwise FP4 fake quantization -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package.  The GPU library never does, and this package imports
nothing from it: the two share no code.

Everything here is numpy on the host.  BF16 tensors are passed as numpy
uint16 arrays holding the raw BF16 bit patterns.  The arithmetic lives in
fq_oracle.c (plain scalar C, each step cited there); this module only
marshals arrays and expresses the transposed-axis variant by its definition:
quantizing along columns is quantizing the transpose along rows, with codes
and scales kept in the transposed layout and y transposed back.

Formats (this package's own names):
  "mx"        MXFP4: 1x32 groups, E8M0 scale
  "nv_tensor" NVFP4: 1x16 groups, E4M3 scale, FP32 per-tensor outer scale
  "nv_128"    NVFP4 double block: 1x16 E4M3 inner scale, FP32 scale per 128
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

FORMATS = {"mx": 0, "nv_tensor": 1, "nv_128": 2}
ROUNDINGS = {"rne": 0, "sr": 1}
BLOCK = {"mx": 32, "nv_tensor": 16, "nv_128": 16}

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        path = _build.ensure_built()
        L = ctypes.CDLL(path)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f32p = ctypes.POINTER(ctypes.c_float)
        i64 = ctypes.c_int64
        L.fqo_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.fqo_bf16_to_f32.restype = ctypes.c_float
        L.fqo_f32_to_bf16.argtypes = [ctypes.c_float]
        L.fqo_f32_to_bf16.restype = ctypes.c_uint16
        L.fqo_e2m1_decode.argtypes = [ctypes.c_int]
        L.fqo_e2m1_decode.restype = ctypes.c_double
        L.fqo_e2m1_rne.argtypes = [ctypes.c_float]
        L.fqo_e2m1_rne.restype = ctypes.c_int
        L.fqo_e2m1_sr.argtypes = [ctypes.c_float, ctypes.c_uint16]
        L.fqo_e2m1_sr.restype = ctypes.c_int
        L.fqo_e8m0_decode.argtypes = [ctypes.c_uint8]
        L.fqo_e8m0_decode.restype = ctypes.c_float
        L.fqo_mx_scale_code.argtypes = [ctypes.c_float]
        L.fqo_mx_scale_code.restype = ctypes.c_uint8
        L.fqo_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.fqo_e4m3_decode.restype = ctypes.c_double
        L.fqo_e4m3_encode.argtypes = [ctypes.c_float]
        L.fqo_e4m3_encode.restype = ctypes.c_uint8
        L.fqo_philox4x32_10.argtypes = [ctypes.POINTER(ctypes.c_uint32),
                                        ctypes.POINTER(ctypes.c_uint32),
                                        ctypes.POINTER(ctypes.c_uint32)]
        L.fqo_philox4x32_10.restype = None
        L.fqo_r16.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.fqo_r16.restype = ctypes.c_uint16
        L.fqo_nv_outer_scale.argtypes = [ctypes.c_float]
        L.fqo_nv_outer_scale.restype = ctypes.c_float
        L.fqo_absmax.argtypes = [u16p, i64]
        L.fqo_absmax.restype = ctypes.c_float
        L.fqo_quantize_rows.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                        u16p, i64, i64, u8p, u8p, f32p, u16p, u8p,
                                        ctypes.c_int]
        L.fqo_quantize_rows.restype = ctypes.c_int
        L.fqo_quantize_rows_at.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                           ctypes.c_uint64, u16p, i64, i64, u8p, u8p, f32p,
                                           u16p, u8p, ctypes.c_int]
        L.fqo_quantize_rows_at.restype = ctypes.c_int
        L.fqo_dequantize_rows.argtypes = [ctypes.c_int, u8p, u8p, f32p, i64, i64,
                                          u16p, ctypes.c_int]
        L.fqo_dequantize_rows.restype = ctypes.c_int
        L.fqo_ste_backward_rows.argtypes = [ctypes.c_int, u16p, u8p, f32p, u16p,
                                            i64, i64, u16p, ctypes.c_int]
        L.fqo_ste_backward_rows.restype = ctypes.c_int
        L.fqo_rht_sign_bit.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.fqo_rht_sign_bit.restype = ctypes.c_int
        L.fqo_hadamard_rows.argtypes = [u16p, i64, i64, ctypes.c_int, ctypes.c_uint64,
                                        ctypes.c_float, u16p, ctypes.c_int]
        L.fqo_hadamard_rows.restype = ctypes.c_int
        L.fqo_quantize_rows_retain.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                               u16p, i64, i64, u8p, f32p, u8p, u8p, f32p,
                                               u16p, ctypes.c_int]
        L.fqo_quantize_rows_retain.restype = ctypes.c_int
        L.fqo_fp8_fake.argtypes = [u16p, f32p, i64, u16p, u8p]
        L.fqo_fp8_fake.restype = ctypes.c_int
        L.fqo_max_threads.argtypes = []
        L.fqo_max_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None, ctype):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# --------------------------------------------------------------------------
# scalar helpers (exposed for the pins)
# --------------------------------------------------------------------------

def bf16_to_f32(h: int) -> float:
    return lib().fqo_bf16_to_f32(h)


def f32_to_bf16(f: float) -> int:
    return lib().fqo_f32_to_bf16(f)


def e2m1_decode(code: int) -> float:
    return lib().fqo_e2m1_decode(code)


def e2m1_rne(a: float) -> int:
    return lib().fqo_e2m1_rne(a)


def e2m1_sr(a: float, r: int) -> int:
    return lib().fqo_e2m1_sr(a, r)


def e8m0_decode(code: int) -> float:
    return lib().fqo_e8m0_decode(code)


def mx_scale_code(amax: float) -> int:
    return lib().fqo_mx_scale_code(amax)


def e4m3_decode(code: int) -> float:
    return lib().fqo_e4m3_decode(code)


def e4m3_encode(v: float) -> int:
    return lib().fqo_e4m3_encode(v)


def nv_outer_scale(amax: float) -> float:
    return lib().fqo_nv_outer_scale(amax)


def philox4x32_10(counter, key):
    c = (ctypes.c_uint32 * 4)(*counter)
    k = (ctypes.c_uint32 * 2)(*key)
    o = (ctypes.c_uint32 * 4)()
    lib().fqo_philox4x32_10(c, k, o)
    return list(o)


def r16(seed: int, n: int) -> int:
    return lib().fqo_r16(seed, n)


# --------------------------------------------------------------------------
# tensor-level calls
# --------------------------------------------------------------------------

def _rows_quantize(fmt: str, rounding: str, seed: int, x: np.ndarray,
                   nthreads: int, index_base: int = 0):
    R, C = x.shape
    B = BLOCK[fmt]
    codes = np.zeros((R, C // 2), np.uint8)
    scales = np.zeros((R, C // B), np.uint8)
    if fmt == "nv_tensor":
        outer = np.zeros((1,), np.float32)
    elif fmt == "nv_128":
        outer = np.zeros((R, C // 128), np.float32)
    else:
        outer = None
    y = np.zeros((R, C), np.uint16)
    clip = np.zeros((R, C), np.uint8)
    rc = lib().fqo_quantize_rows_at(FORMATS[fmt], ROUNDINGS[rounding], seed, index_base,
                                 _ptr(x, ctypes.c_uint16), R, C,
                                 _ptr(codes, ctypes.c_uint8),
                                 _ptr(scales, ctypes.c_uint8),
                                 _ptr(outer, ctypes.c_float),
                                 _ptr(y, ctypes.c_uint16),
                                 _ptr(clip, ctypes.c_uint8), nthreads)
    if rc != 0:
        raise ValueError(f"oracle: shape {x.shape} cannot be blocked for {fmt}")
    return codes, scales, outer, y, clip


def fake_quant(x: np.ndarray, fmt: str, rounding: str = "rne", axis: str = "row",
               seed: int = 0, nthreads: int | None = None, index_base: int = 0) -> dict:
    """Quantize and dequantize a [R, C] BF16 tensor (uint16 bit patterns).

    axis="row": 1xB groups along each row.  codes [R, C/2], scales [R, C/B],
    outer (nv_tensor: [1]; nv_128: [R, C/128]), y [R, C].
    axis="col": 1xB groups along each column, i.e. the row quantization of
    x^T.  codes [C, R/2], scales [C, R/B], outer [1] or [C, R/128] (the
    transposed layout); y [R, C] in the layout of x; the stochastic-rounding
    index of element (i, j) is j * R + i.
    Also returns clip (1 where the element was clipped), in the layout of y.
    index_base is added to every stochastic-rounding index: for a sample of
    whole rows (row axis) or of one whole column (column axis) cut from a
    larger tensor, the flat index of the sample's first element in that
    tensor (r0 * C_full, resp. c * R).  A per-tensor scale is then the
    sample's own.
    """
    x = np.ascontiguousarray(x, dtype=np.uint16)
    assert x.ndim == 2
    n = default_threads() if nthreads is None else nthreads
    src = x if axis == "row" else np.ascontiguousarray(x.T)
    codes, scales, outer, y, clip = _rows_quantize(fmt, rounding, seed, src, n, index_base)
    if axis == "col":
        y = np.ascontiguousarray(y.T)
        clip = np.ascontiguousarray(clip.T)
    return {"codes": codes, "scales": scales, "outer": outer, "y": y, "clip": clip}


def dequantize(codes: np.ndarray, scales: np.ndarray, outer, fmt: str,
               shape: tuple[int, int], axis: str = "row",
               nthreads: int | None = None) -> np.ndarray:
    """Inverse of fake_quant's encode step: y [R, C] for x of shape `shape`."""
    R, C = shape
    QR, QC = (R, C) if axis == "row" else (C, R)
    n = default_threads() if nthreads is None else nthreads
    y = np.zeros((QR, QC), np.uint16)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    outer = None if outer is None else np.ascontiguousarray(outer, dtype=np.float32)
    rc = lib().fqo_dequantize_rows(FORMATS[fmt], _ptr(codes, ctypes.c_uint8),
                                   _ptr(scales, ctypes.c_uint8),
                                   _ptr(outer, ctypes.c_float), QR, QC,
                                   _ptr(y, ctypes.c_uint16), n)
    if rc != 0:
        raise ValueError("oracle: bad shape for dequantize")
    return y if axis == "row" else np.ascontiguousarray(y.T)


def ste_backward(x: np.ndarray, scales: np.ndarray, outer, dy: np.ndarray,
                 fmt: str, axis: str = "row", nthreads: int | None = None) -> np.ndarray:
    """dx = dy where the forward did not clip x, else +0 (layout of x)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    dy = np.ascontiguousarray(dy, dtype=np.uint16)
    n = default_threads() if nthreads is None else nthreads
    if axis == "col":
        x = np.ascontiguousarray(x.T)
        dy = np.ascontiguousarray(dy.T)
    QR, QC = x.shape
    dx = np.zeros((QR, QC), np.uint16)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    outer = None if outer is None else np.ascontiguousarray(outer, dtype=np.float32)
    rc = lib().fqo_ste_backward_rows(FORMATS[fmt], _ptr(x, ctypes.c_uint16),
                                     _ptr(scales, ctypes.c_uint8),
                                     _ptr(outer, ctypes.c_float),
                                     _ptr(dy, ctypes.c_uint16), QR, QC,
                                     _ptr(dx, ctypes.c_uint16), n)
    if rc != 0:
        raise ValueError("oracle: bad shape for ste_backward")
    return dx if axis == "row" else np.ascontiguousarray(dx.T)


def keep_mask(clip: np.ndarray) -> np.ndarray:
    """Bit-packed STE keep mask of a fake_quant clip array, in the layout of x.

    The straight-through gradient passes where the forward kept the element,
    i.e. where a = RN(|x| / s_eff) <= 6 ("Resumo Tecnico: TetraJet-v2", sec.
    2.A, the clipping that the gradient must respect; the same test as
    ste_backward).  Byte (r, c // 8) holds elements (r, 8*(c//8)) .. +7, bit
    c mod 8 set when element (r, c) was kept.  C must be a multiple of 8.
    """
    clip = np.ascontiguousarray(clip, dtype=np.uint8)
    assert clip.ndim == 2 and clip.shape[1] % 8 == 0
    return np.packbits(clip == 0, axis=1, bitorder="little")


def ste_backward_mask(keep: np.ndarray, dy: np.ndarray) -> np.ndarray:
    """dx = dy where the keep bit of the element is set, else +0 (BF16 bits)."""
    dy = np.ascontiguousarray(dy, dtype=np.uint16)
    bits = np.unpackbits(np.ascontiguousarray(keep, dtype=np.uint8), axis=1,
                         bitorder="little")
    assert bits.shape == dy.shape
    return np.where(bits == 1, dy, np.uint16(0)).astype(np.uint16)


# --------------------------------------------------------------------------
# TetraJet-v2 sec. 2.B (OsciReset) and sec. 2.C (static outlier retention)
# --------------------------------------------------------------------------

def osci_state(n: int) -> dict:
    """Per-element OsciReset state for n weights: previous master weight
    (FP32), previous quantized value (BF16 bits) and the two distances (FP32)."""
    return {"w_prev": np.zeros(n, np.float32), "q_prev": np.zeros(n, np.uint16),
            "dist_m": np.zeros(n, np.float32), "dist_q": np.zeros(n, np.float32)}


def osci_track(w: np.ndarray, q: np.ndarray, st: dict, first: bool) -> None:
    """One training step of the oscillation tracker ("Resumo Tecnico:
    TetraJet-v2", sec. 2.B, detection): the distance the master weight w
    (FP32) and its quantized value q (BF16 bits, the fake-quantized weight the
    forward used) travelled since the previous step is added to dist_m and
    dist_q.  Every difference and every sum is one FP32 operation (numpy
    float32 arithmetic rounds each to nearest).  first=True starts the
    trajectory: it records w and q and clears the distances."""
    w = np.asarray(w, np.float32).reshape(-1)
    q = np.asarray(q, np.uint16).reshape(-1)
    if first:
        st["dist_m"][:] = 0
        st["dist_q"][:] = 0
    else:
        qf = bf16_bits_to_f64(q).astype(np.float32)
        qp = bf16_bits_to_f64(st["q_prev"]).astype(np.float32)
        st["dist_m"][:] = st["dist_m"] + np.abs(w - st["w_prev"])
        st["dist_q"][:] = st["dist_q"] + np.abs(qf - qp)
    st["w_prev"][:] = w
    st["q_prev"][:] = q


E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def e2m1_bin_centres() -> list[float]:
    """Centre of the quantization bin of each E2M1 magnitude code m = 0..7.

    "Resumo Tecnico: TetraJet-v2", sec. 2.B (mechanism) resets an oscillating
    master weight to the centre of its current quantization bin.  The bin of
    grid value g_m is the interval of scaled magnitudes that round to it: from
    the midpoint with the grid value below to the midpoint with the one above.
    READINGS: the bin of 0 holds both signs ([-0.25, 0.25], centre 0); E2M1
    stops at 6, so the top bin (from 5 up) is closed at 7, the midpoint with
    8, the value that follows 4 and 6 in the format's exponent progression,
    which puts its centre on 6 itself (also the largest magnitude the clipped
    straight-through gradient still passes).
    """
    g = list(E2M1_GRID) + [8.0]
    out = []
    for m in range(8):
        hi = (g[m] + g[m + 1]) / 2
        lo = -hi if m == 0 else (g[m - 1] + g[m]) / 2
        out.append((lo + hi) / 2)
    return out


def element_code_and_scale(codes: np.ndarray, scales: np.ndarray, outer, fmt: str,
                           shape: tuple[int, int], axis: str = "row"):
    """Per element of x [R, C]: its E2M1 code (uint8) and effective block scale
    s_eff (float32), read from quantizer outputs in the layout of `axis`
    (MXFP4: 2^(code - 127); NVFP4: RN32(e4m3(code) * s), s the per-tensor or
    128-block outer scale)."""
    R, C = shape
    QR, QC = (R, C) if axis == "row" else (C, R)
    B = BLOCK[fmt]
    packed = np.asarray(codes, np.uint8).reshape(QR, QC // 2)
    code = np.empty((QR, QC), np.uint8)
    code[:, 0::2] = packed & 15
    code[:, 1::2] = packed >> 4
    sc = np.repeat(np.asarray(scales, np.uint8).reshape(QR, QC // B), B, axis=1)
    if fmt == "mx":
        table = np.array([e8m0_decode(c) for c in range(255)] + [np.nan], np.float32)
        s_eff = table[sc]
    else:
        table = np.array([e4m3_decode(c) for c in range(256)], np.float64).astype(np.float32)
        if fmt == "nv_tensor":
            s = np.float32(np.asarray(outer, np.float32).reshape(-1)[0])
        else:
            s = np.repeat(np.asarray(outer, np.float32).reshape(QR, QC // 128), 128, axis=1)
        s_eff = (table[sc] * s).astype(np.float32)        # one FP32 rounding
    if axis == "col":
        code, s_eff = code.T, s_eff.T
    return np.ascontiguousarray(code), np.ascontiguousarray(s_eff)


def bin_centre_values(codes: np.ndarray, scales: np.ndarray, outer, fmt: str,
                      shape: tuple[int, int], axis: str = "row") -> np.ndarray:
    """FP32 [R, C]: sign(code) * RN32(c_m * s_eff), the centre of each element's
    current quantization bin in the units of x (c_m from e2m1_bin_centres,
    exact in FP32; the sign of the code is kept, so code 8 gives -0.0)."""
    code, s_eff = element_code_and_scale(codes, scales, outer, fmt, shape, axis)
    c = np.array(e2m1_bin_centres(), np.float32)[code & 7]
    mag = (c * s_eff).astype(np.float32)
    return np.where(code >= 8, -mag, mag).astype(np.float32)


def osci_reset(w: np.ndarray, q: np.ndarray, st: dict, tau: float, target: str = "centre",
               quant: dict | None = None, fmt: str | None = None, axis: str = "row"):
    """The OsciReset check (sec. 2.B, mechanism), called by the training loop
    when the learning rate is low.  The oscillation risk is dist_q / dist_m;
    READING: an element oscillates when dist_q > RN32(tau * dist_m) (so a
    quantized value that moved while the master weight did not counts, and
    one that never moved does not).

    target "centre" (the page's mechanism): an oscillating master weight goes
    to the centre of its current quantization bin (bin_centre_values), read
    from `quant`, the codes / scales / outer of the quantization that gave q
    (fake_quant's output for w's BF16 copy, format fmt, along `axis`); w is
    then [R, C] shaped like that quantization's input.  target "grid": it
    goes to its quantized value q itself (the grid point its bin maps to).

    A check starts a new window: the distances restart at 0 and the
    trajectory continues from the (reset) weights.  Returns the new w (flat)
    and the boolean mask of reset elements."""
    shape = np.shape(w)
    w = np.array(w, np.float32).reshape(-1)
    q = np.asarray(q, np.uint16).reshape(-1)
    osc = st["dist_q"] > (np.float32(tau) * st["dist_m"])
    if target == "grid":
        w[osc] = bf16_bits_to_f64(q[osc]).astype(np.float32)
    elif target == "centre":
        cv = bin_centre_values(quant["codes"], quant["scales"], quant["outer"], fmt,
                               shape, axis).reshape(-1)
        w[osc] = cv[osc]
    else:
        raise ValueError(f"unknown reset target {target!r}")
    st["w_prev"][:] = w
    st["q_prev"][:] = q
    st["dist_m"][:] = 0
    st["dist_q"][:] = 0
    return w, osc


def channel_absmax(x: np.ndarray, running: np.ndarray | None = None) -> np.ndarray:
    """Per-channel (per-column) maximum |x| of a BF16 [R, C] tensor, as BF16
    magnitude bits (uint32), folded into `running` if given ("Resumo Tecnico:
    TetraJet-v2", sec. 2.C: outlier channels are identified by their norms over
    a calibration window; READING: the norm is the maximum magnitude, which is
    exact and independent of summation order)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    m = (x & np.uint16(0x7FFF)).max(axis=0).astype(np.uint32)
    return m if running is None else np.maximum(running, m)


def select_channels(amax_bits: np.ndarray, k: int):
    """The k channels with the largest calibration magnitude (ties: lower
    channel index first) and their FP8 scales s_c = RN32(amax_c / 448)
    (sec. 2.C: the top p% channels stay in FP8, E4M3's largest value 448).
    Returns (retain [C] bool, chan_scale [C] float32, 0 where not retained)."""
    a = np.asarray(amax_bits, np.uint32)
    C = a.size
    order = sorted(range(C), key=lambda c: (-int(a[c]), c))
    retain = np.zeros(C, bool)
    retain[order[:k]] = True
    amax = bf16_bits_to_f64(a.astype(np.uint16)).astype(np.float32)
    scale = np.where(retain, amax / np.float32(448.0), np.float32(0)).astype(np.float32)
    return retain, scale


def fp8_fake(x: np.ndarray, scale: np.ndarray):
    """Element-wise FP8 E4M3 fake quantization of BF16 values x under the
    FP32 scales `scale` (same shape): y (BF16 bits) and the clip flag
    (a = |x| / s > 448)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    sc = np.ascontiguousarray(np.broadcast_to(scale, x.shape), dtype=np.float32)
    y = np.empty_like(x)
    clip = np.empty(x.shape, np.uint8)
    lib().fqo_fp8_fake(_ptr(x, ctypes.c_uint16), _ptr(sc, ctypes.c_float), x.size,
                       _ptr(y, ctypes.c_uint16), _ptr(clip, ctypes.c_uint8))
    return y, clip


def fake_quant_retained(x: np.ndarray, fmt: str, retain: np.ndarray, chan_scale: np.ndarray,
                        rounding: str = "rne", axis: str = "row", seed: int = 0,
                        nthreads: int | None = None) -> dict:
    """Fake quantization with static outlier-channel retention ("Resumo
    Tecnico: TetraJet-v2", sec. 2.C) along either axis and in every format.

    The channels are the columns of x [R, C] (retain [C] bool, chan_scale [C]
    FP32).  READING (the same as fqo_quantize_rows_retain's on the row axis):
    a retained element takes no part in any FP4 maximum (block, 128-block or
    tensor) and carries FP4 code 0; its value is its FP8 fake quantization.
    That is exactly the plain quantizer applied to x with the retained columns
    set to +0, with the FP8 values put in their place: along the row axis the
    retained columns drop out of the blocks they share with other columns;
    along the column axis every block of a retained column is empty.  Returns
    codes / scales / outer of the FP4 part (layouts of fake_quant), y, and
    clip (FP4 rule for the rest, FP8 rule, a > 448, for retained elements)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    ret = np.asarray(retain, bool)
    cs = np.asarray(chan_scale, np.float32)
    xz = x.copy()
    xz[:, ret] = 0
    q = fake_quant(xz, fmt, rounding, axis, seed, nthreads)
    y8, clip8 = fp8_fake(x[:, ret], np.broadcast_to(cs[ret], (x.shape[0], int(ret.sum()))))
    y = q["y"].copy()
    y[:, ret] = y8
    # the FP4 straight-through test recomputed from x and the stored scales,
    # as ste_backward does, then the FP8 test for the retained columns
    ones = np.full(x.shape, 0x3F80, dtype=np.uint16)
    clip = (ste_backward(x, q["scales"], q["outer"], ones, fmt, axis, nthreads) == 0)
    clip = clip.astype(np.uint8)
    clip[:, ret] = clip8
    return {"codes": q["codes"], "scales": q["scales"], "outer": q["outer"], "y": y,
            "clip": clip}


def fake_quant_retain(x: np.ndarray, fmt: str, retain: np.ndarray, chan_scale: np.ndarray,
                      rounding: str = "rne", seed: int = 0,
                      nthreads: int | None = None) -> dict:
    """Row-axis fake quantization in which the retained channels (columns)
    are FP8 E4M3 with their own scale and the rest FP4 (fqo_quantize_rows_retain).
    fmt "mx" or "nv_128"."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    R, C = x.shape
    B = BLOCK[fmt]
    ret = np.ascontiguousarray(np.asarray(retain).astype(np.uint8))
    sc = np.ascontiguousarray(chan_scale, dtype=np.float32)
    codes = np.zeros((R, C // 2), np.uint8)
    scales = np.zeros((R, C // B), np.uint8)
    outer = np.zeros((R, C // 128), np.float32) if fmt == "nv_128" else None
    y = np.zeros((R, C), np.uint16)
    n = default_threads() if nthreads is None else nthreads
    rc = lib().fqo_quantize_rows_retain(FORMATS[fmt], ROUNDINGS[rounding], seed,
                                        _ptr(x, ctypes.c_uint16), R, C,
                                        _ptr(ret, ctypes.c_uint8), _ptr(sc, ctypes.c_float),
                                        _ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8),
                                        _ptr(outer, ctypes.c_float), _ptr(y, ctypes.c_uint16), n)
    if rc != 0:
        raise ValueError(f"oracle: {fmt} {x.shape} cannot be quantized with retained channels")
    return {"codes": codes, "scales": scales, "outer": outer, "y": y}


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    """Exact widening of BF16 bit patterns to float64."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def qlinear(x: np.ndarray, w: np.ndarray, fmt_x: str = "nv_tensor",
            fmt_w: str = "nv_tensor", rounding_x: str = "rne",
            rounding_w: str = "rne", seed_x: int = 0, seed_w: int = 0,
            nthreads: int | None = None, retain=None, chan_scale=None) -> dict:
    """QAT linear forward: Y = FQ(X) @ FQ(W).

    X [M, K] is quantized in groups along K (its rows), W [K, N] in groups
    along K (its columns, the transposed axis).  Y is the float64 product of
    the two dequantized BF16 tensors (numpy matmul as the contraction step).
    With retain / chan_scale the activation's retained channels (columns of X)
    are FP8 (fake_quant_retained), the rest FP4 ("Resumo Tecnico:
    TetraJet-v2", sec. 2.C, forward pass).
    """
    if retain is None:
        fx = fake_quant(x, fmt_x, rounding_x, "row", seed_x, nthreads)
    else:
        fx = fake_quant_retained(x, fmt_x, retain, chan_scale, rounding_x, "row", seed_x,
                                 nthreads)
    fw = fake_quant(w, fmt_w, rounding_w, "col", seed_w, nthreads)
    Y = bf16_bits_to_f64(fx["y"]) @ bf16_bits_to_f64(fw["y"])
    return {"xhat": fx["y"], "what": fw["y"], "y": Y}


def _clip_keep(x: np.ndarray, q: dict, fmt: str, axis: str) -> np.ndarray:
    """1.0 where the forward kept x (a <= 6), 0.0 where it clipped."""
    ones = np.full(x.shape, 0x3F80, dtype=np.uint16)      # BF16 1.0
    return bf16_bits_to_f64(ste_backward(x, q["scales"], q["outer"], ones, fmt, axis))


def qlinear_bwd(x: np.ndarray, w: np.ndarray, dy: np.ndarray, fmt_x: str = "nv_tensor",
                fmt_w: str = "nv_tensor", fmt_g: str = "nv_128", rounding_g: str = "sr",
                seed_g: int = 0, rounding_x: str = "rne", rounding_w: str = "rne",
                seed_x: int = 0, seed_w: int = 0, rht_block: int = 0, rht_seed: int = 0,
                nthreads: int | None = None, retain=None, chan_scale=None) -> dict:
    """QAT linear backward of Y = FQ(X) @ FQ(W) (TetraJet-v2 sec. 2.A).

    X_hat = FQ(X) along K and W_hat = FQ(W) along K are the forward operands.
    Each backward product quantizes both of its operands along its own
    contraction axis with fmt_g / rounding_g:
        dX = keep_X * (Q(dY, along N) @ Q(W_hat, along N)^T)     [M, K]
        dW = keep_W * (Q(X_hat, along M)^T @ Q(dY, along M))     [K, N]
    with Philox keys seed_g + 0, + 1, + 2, + 3 for the four Q in that order,
    and keep_* the STE masks of the forward (1 where a <= 6).  With rht_block
    16 or 128 each Q's input is first rotated along that Q's axis by the
    random Hadamard transform (seed rht_seed; TetraJet-v2 sec. 2.C).  With
    retain / chan_scale the activation's retained channels are FP8 in X_hat
    and in Q(X_hat, along M), and keep_X uses the FP8 clip test for them
    (sec. 2.C: the channels stay in higher precision in the forward and the
    backward pass).  The products are float64 (numpy matmul as the
    contraction step).
    """
    if retain is None:
        fx = fake_quant(x, fmt_x, rounding_x, "row", seed_x, nthreads)
    else:
        assert not rht_block, "retention with the rotated backward is not defined here"
        fx = fake_quant_retained(x, fmt_x, retain, chan_scale, rounding_x, "row", seed_x,
                                 nthreads)
    fw = fake_quant(w, fmt_w, rounding_w, "col", seed_w, nthreads)
    m64 = (1 << 64) - 1
    rot = (lambda t, ax: hadamard(t, rht_block, ax, rht_seed, nthreads)) if rht_block else \
        (lambda t, ax: t)
    q_dy_n = fake_quant(rot(dy, "row"), fmt_g, rounding_g, "row", (seed_g + 0) & m64, nthreads)
    q_w_n = fake_quant(rot(fw["y"], "row"), fmt_g, rounding_g, "row", (seed_g + 1) & m64,
                       nthreads)
    if retain is None:
        q_x_m = fake_quant(rot(fx["y"], "col"), fmt_g, rounding_g, "col", (seed_g + 2) & m64,
                           nthreads)
    else:
        # the retained channels stay FP8 in the backward too (sec. 2.C)
        q_x_m = fake_quant_retained(fx["y"], fmt_g, retain, chan_scale, rounding_g, "col",
                                    (seed_g + 2) & m64, nthreads)
    q_dy_m = fake_quant(rot(dy, "col"), fmt_g, rounding_g, "col", (seed_g + 3) & m64, nthreads)
    dx_raw = bf16_bits_to_f64(q_dy_n["y"]) @ bf16_bits_to_f64(q_w_n["y"]).T
    dw_raw = bf16_bits_to_f64(q_x_m["y"]).T @ bf16_bits_to_f64(q_dy_m["y"])
    keep_x = _clip_keep(x, fx, fmt_x, "row") if retain is None else \
        (1.0 - fx["clip"].astype(np.float64))
    keep_w = _clip_keep(w, fw, fmt_w, "col")
    return {"dx": keep_x * dx_raw, "dw": keep_w * dw_raw, "xhat": fx["y"], "what": fw["y"],
            "q_dy_n": q_dy_n["y"], "q_w_n": q_w_n["y"], "q_x_m": q_x_m["y"],
            "q_dy_m": q_dy_m["y"], "keep_x": keep_x, "keep_w": keep_w}


# FP32 value nearest to 1/sqrt(n): 0.25 for n = 16; for n = 128 the bits
# 0x3DB504F3 (the test suite checks that no other FP32 value is nearer).
RHT_SCALE_BITS = {16: 0x3E800000, 128: 0x3DB504F3}


def rht_scale(n: int) -> float:
    return float(np.array([RHT_SCALE_BITS[n]], dtype=np.uint32).view(np.float32)[0])


def rht_sign_bit(seed: int, j: int) -> int:
    """1 where position j of the random Hadamard transform flips sign."""
    return lib().fqo_rht_sign_bit(seed, j)


def hadamard(x: np.ndarray, block: int, axis: str = "row", seed: int = 0,
             nthreads: int | None = None) -> np.ndarray:
    """Random Hadamard transform of a [R, C] BF16 tensor (uint16 bits) in
    blocks of `block` (16 or 128) consecutive elements along `axis`; BF16
    result in the layout of x.  axis="col" is the row transform of x^T."""
    n = default_threads() if nthreads is None else nthreads
    src = np.ascontiguousarray(x if axis == "row" else x.T, dtype=np.uint16)
    R, C = src.shape
    y = np.empty_like(src)
    rc = lib().fqo_hadamard_rows(_ptr(src, ctypes.c_uint16), R, C, block, seed,
                                 rht_scale(block), _ptr(y, ctypes.c_uint16), n)
    if rc != 0:
        raise ValueError(f"hadamard: unsupported shape {src.shape} for block {block}")
    return y if axis == "row" else np.ascontiguousarray(y.T)
