"""The C-ABI library loads, exports every symbol include/fq.h declares, and
rejects bad arguments with the documented status before touching the device.

No call here reaches a kernel launch: every call either returns a constant
(presets, sizes, strings) or fails validation.  The pointers passed are fake
but aligned (validation never dereferences them).
"""
import ctypes
import os
import re

import pytest

import fp4_block_quantization_fq_amd as fq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "fq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(fq_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fq.LIB_PATH):
        pytest.skip("libfq.so not built")
    return fq.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 12, names
    assert sorted(fq.EXPORTED) == names
    for n in names:
        assert hasattr(L, n), n


def test_presets_are_the_one_line_switch(L):
    mx, nv = L.fq_desc_mxfp4(), L.fq_desc_nvfp4()
    assert (mx.block_size, mx.scale_type, mx.outer, mx.rounding, mx.axis, mx.seed) == (32, 0, 0, 0, 0, 0)
    assert (nv.block_size, nv.scale_type, nv.outer, nv.rounding, nv.axis, nv.seed) == (16, 1, 1, 0, 0, 0)
    assert ctypes.sizeof(fq.FqDesc) == 32


def test_workspace_sizes(L):
    mx, nv = fq.fq_desc_mxfp4(), fq.fq_desc_nvfp4()
    nv128 = fq.fq_desc_nvfp4(outer=fq.FQ_OUTER_BLOCK128)
    assert L.fq_workspace_size(ctypes.byref(mx), 1024, 4096) == 0
    assert L.fq_workspace_size(ctypes.byref(nv), 1024, 4096) == 4096
    assert L.fq_workspace_size(ctypes.byref(nv128), 1024, 4096) == 0
    bad = fq.fq_desc_mxfp4()
    bad.block_size = 16
    assert L.fq_workspace_size(ctypes.byref(bad), 1024, 4096) == 0
    M, K, N = 8192, 2880, 5760
    want = (M * K * 2 + 255) // 256 * 256 + (N * K * 2 + 255) // 256 * 256 + 8192
    assert L.fq_qlinear_workspace_size(ctypes.byref(nv), ctypes.byref(nv), M, K, N) == want


P = ctypes.c_void_p


def fake(addr=0x10000):
    return P(addr)


def call_quant(L, d, rows=64, cols=64, x=fake(), codes=fake(), scales=fake(), outer=fake(),
               ws=fake(), ws_bytes=4096):
    return L.fq_quantize(ctypes.byref(d) if d is not None else None, x, rows, cols, codes,
                         scales, outer, ws, ws_bytes, None)


def test_quantize_validation(L):
    mx = fq.fq_desc_mxfp4()
    nv = fq.fq_desc_nvfp4()
    assert call_quant(L, None) == fq.FQ_ERR_NULL
    assert call_quant(L, mx, x=None) == fq.FQ_ERR_NULL
    assert call_quant(L, mx, codes=None) == fq.FQ_ERR_NULL
    assert call_quant(L, nv, outer=None) == fq.FQ_ERR_NULL
    assert call_quant(L, nv, ws=None) == fq.FQ_ERR_NULL
    assert call_quant(L, mx, x=fake(0x10008)) == fq.FQ_ERR_ALIGN
    assert call_quant(L, nv, outer=fake(0x10002)) == fq.FQ_ERR_ALIGN
    assert call_quant(L, nv, ws_bytes=4095) == fq.FQ_ERR_WORKSPACE
    assert call_quant(L, mx, cols=48) == fq.FQ_ERR_SHAPE           # not a multiple of 32
    assert call_quant(L, mx, rows=0) == fq.FQ_ERR_SHAPE
    assert call_quant(L, mx, rows=1 << 20, cols=1 << 15) == fq.FQ_ERR_SHAPE   # > 2^34
    nv128 = fq.fq_desc_nvfp4(outer=fq.FQ_OUTER_BLOCK128)
    assert call_quant(L, nv128, cols=64) == fq.FQ_ERR_SHAPE        # not a multiple of 128
    col = fq.fq_desc_nvfp4(axis=fq.FQ_AXIS_COL)
    assert call_quant(L, col, rows=24, cols=64) == fq.FQ_ERR_SHAPE  # rows not multiple of 16
    assert call_quant(L, col, rows=32, cols=20) == fq.FQ_ERR_SHAPE  # cols not multiple of 8
    for field, val in [("block_size", 8), ("scale_type", 1), ("outer", 1), ("rounding", 2),
                       ("axis", 3), ("reserved", 1)]:
        d = fq.fq_desc_mxfp4()
        setattr(d, field, val)
        assert call_quant(L, d) == fq.FQ_ERR_DESC, field
    msg = L.fq_last_error().decode()
    assert "reserved" in msg


def test_dimension_limits(L):
    """Each dimension below 2^31 (the kernels take 32-bit rows and columns and
    the products int tile indexes), and no overflow of rows * cols for huge
    dimensions whose product would wrap."""
    mx = fq.fq_desc_mxfp4()
    big = 1 << 31                                  # rows * cols = 2^31 <= 2^34
    assert call_quant(L, mx, rows=1, cols=big) == fq.FQ_ERR_SHAPE
    assert call_quant(L, fq.fq_desc_mxfp4(axis=fq.FQ_AXIS_COL), rows=big, cols=8) == fq.FQ_ERR_SHAPE
    assert call_quant(L, mx, rows=1 << 34, cols=1 << 34) == fq.FQ_ERR_SHAPE   # product wraps int64
    assert L.fq_hadamard(fake(), 1, big, fq.FQ_AXIS_ROW, 128, 0, fake(0x20000), None) == fq.FQ_ERR_SHAPE
    assert "2^31" in L.fq_last_error().decode()
    assert L.fq_ste_backward_mask(fake(), fake(), 1, big, fake(), None) == fq.FQ_ERR_SHAPE
    assert L.fq_channel_absmax(fake(), 1, big, fake(), None) == fq.FQ_ERR_SHAPE
    nv, col = fq.fq_desc_nvfp4(), fq.fq_desc_nvfp4(axis=fq.FQ_AXIS_COL)
    assert L.fq_qlinear_fwd(ctypes.byref(nv), ctypes.byref(col), fake(), fake(), 1, big, 8,
                            fake(), fake(), 1 << 40, None) == fq.FQ_ERR_SHAPE
    assert L.fq_qlinear_workspace_size(ctypes.byref(nv), ctypes.byref(col), 1, big, 8) == 0


def test_other_entry_points_validate(L):
    mx = fq.fq_desc_mxfp4()
    nv = fq.fq_desc_nvfp4()
    assert L.fq_dequantize(ctypes.byref(mx), fake(), None, None, 64, 64, fake(), None) == fq.FQ_ERR_NULL
    assert L.fq_dequantize(ctypes.byref(nv), fake(), fake(), None, 64, 64, fake(), None) == fq.FQ_ERR_NULL
    assert L.fq_dequantize(ctypes.byref(mx), fake(), fake(), None, 64, 40, fake(), None) == fq.FQ_ERR_SHAPE
    assert L.fq_fake_quant(ctypes.byref(mx), fake(), 64, 64, None, None, None, None, None, 0,
                           None) == fq.FQ_ERR_NULL
    assert L.fq_fake_quant(ctypes.byref(mx), fake(), 64, 64, fake(), fake(0x10001), None, None,
                           None, 0, None) == fq.FQ_ERR_ALIGN
    assert L.fq_fake_quant(ctypes.byref(nv), fake(), 64, 64, fake(), None, None, None, None, 0,
                           None) == fq.FQ_ERR_NULL
    assert L.fq_ste_backward(ctypes.byref(mx), fake(), fake(), None, None, 64, 64, fake(),
                             None) == fq.FQ_ERR_NULL
    assert L.fq_ste_backward(ctypes.byref(nv), fake(), fake(), None, fake(), 64, 64, fake(),
                             None) == fq.FQ_ERR_NULL
    # qlinear: axes must put both blocks along K
    col = fq.fq_desc_nvfp4(axis=fq.FQ_AXIS_COL)
    ws = 1 << 30
    assert L.fq_qlinear_fwd(ctypes.byref(nv), ctypes.byref(nv), fake(), fake(), 128, 128, 128,
                            fake(), fake(), ws, None) == fq.FQ_ERR_DESC
    assert L.fq_qlinear_fwd(ctypes.byref(col), ctypes.byref(col), fake(), fake(), 128, 128, 128,
                            fake(), fake(), ws, None) == fq.FQ_ERR_DESC
    # documented shape rules: K a multiple of 64 (K = 96 is a whole number of
    # NVFP4 blocks but not of the 64-element K step), N a multiple of 8
    assert L.fq_qlinear_fwd(ctypes.byref(nv), ctypes.byref(col), fake(), fake(), 128, 96, 128,
                            fake(), fake(), ws, None) == fq.FQ_ERR_SHAPE
    assert L.fq_qlinear_fwd(ctypes.byref(nv), ctypes.byref(col), fake(), fake(), 128, 128, 132,
                            fake(), fake(), ws, None) == fq.FQ_ERR_SHAPE
    assert L.fq_qlinear_fwd(ctypes.byref(nv), ctypes.byref(col), fake(), fake(), 128, 128, 128,
                            fake(), fake(), 1024, None) == fq.FQ_ERR_WORKSPACE


def test_mask_entry_points_validate(L):
    mx = fq.fq_desc_mxfp4()
    nv = fq.fq_desc_nvfp4()

    def fqm(d, keep, rows=64, cols=64, y=fake(), ws=None, nbytes=0):
        return L.fq_fake_quant_mask(ctypes.byref(d), fake(), rows, cols, y, None, None, None,
                                    keep, ws, nbytes, None)
    assert fqm(mx, None) == fq.FQ_ERR_NULL                     # keep is required
    assert fqm(mx, fake(0x10004)) == fq.FQ_ERR_ALIGN
    assert fqm(mx, fake(), y=None) == fq.FQ_ERR_NULL
    assert fqm(mx, fake(), cols=48) == fq.FQ_ERR_SHAPE         # not a multiple of 32
    assert fqm(nv, fake()) == fq.FQ_ERR_NULL                   # per-tensor needs ws
    assert fqm(nv, fake(), ws=fake(), nbytes=100) == fq.FQ_ERR_WORKSPACE
    col = fq.fq_desc_mxfp4(axis=fq.FQ_AXIS_COL)
    assert fqm(col, fake(), rows=32, cols=20) == fq.FQ_ERR_SHAPE

    def stm(keep=fake(), dy=fake(), rows=64, cols=64, dx=fake()):
        return L.fq_ste_backward_mask(keep, dy, rows, cols, dx, None)
    assert stm(keep=None) == fq.FQ_ERR_NULL
    assert stm(dy=None) == fq.FQ_ERR_NULL
    assert stm(dx=None) == fq.FQ_ERR_NULL
    assert stm(keep=fake(0x10008)) == fq.FQ_ERR_ALIGN
    assert stm(cols=12) == fq.FQ_ERR_SHAPE
    assert stm(cols=0) == fq.FQ_ERR_SHAPE
    assert stm(rows=0) == fq.FQ_ERR_SHAPE
    assert stm(rows=1 << 20, cols=1 << 15) == fq.FQ_ERR_SHAPE   # > 2^34 elements


def test_outcontrol_entry_points_validate(L):
    f = fake
    # OsciReset: n a positive multiple of 4, all state pointers required
    assert L.fq_osci_track(f(), f(), f(), f(), f(), f(), 6, 0, None) == fq.FQ_ERR_SHAPE
    assert L.fq_osci_track(f(), f(), f(), f(), f(), f(), 0, 0, None) == fq.FQ_ERR_SHAPE
    assert L.fq_osci_track(f(), None, f(), f(), f(), f(), 64, 0, None) == fq.FQ_ERR_NULL
    assert L.fq_osci_track(f(0x10004), f(), f(), f(), f(), f(), 64, 0, None) == fq.FQ_ERR_ALIGN
    assert L.fq_osci_track(f(), f(0x10004), f(), f(), f(), f(), 64, 0, None) == fq.FQ_ERR_ALIGN
    # fq_osci_reset(desc, w, q, codes, scales, outer, rows, cols, w_prev, q_prev,
    #               dist_m, dist_q, tau, target, stream)
    mx = fq.fq_desc_mxfp4()
    nv = fq.fq_desc_nvfp4()
    C, G = fq.FQ_OSCI_BIN_CENTRE, fq.FQ_OSCI_GRID_VALUE

    def rst(desc=mx, w=f(), q=f(), codes=f(), scales=f(), outer=None, rows=2, cols=32,
            tau=2.0, target=C):
        d = None if desc is None else ctypes.byref(desc)
        return L.fq_osci_reset(d, w, q, codes, scales, outer, rows, cols, f(), f(), f(), f(),
                               ctypes.c_float(tau), target, None)

    assert rst(q=None) == fq.FQ_ERR_NULL
    for bad in (-1.0, float("nan"), float("inf")):
        assert rst(tau=bad) == fq.FQ_ERR_DESC, bad
    assert rst(target=2) == fq.FQ_ERR_DESC
    assert rst(cols=30) == fq.FQ_ERR_SHAPE                  # cols % 4
    assert rst(rows=0) == fq.FQ_ERR_SHAPE
    assert rst(cols=36) == fq.FQ_ERR_SHAPE                  # MXFP4 row blocks of 32
    assert rst(desc=None) == fq.FQ_ERR_NULL                 # the centre needs the format
    assert rst(codes=None) == fq.FQ_ERR_NULL
    assert rst(scales=None) == fq.FQ_ERR_NULL
    assert rst(desc=nv, cols=48) == fq.FQ_ERR_NULL         # NVFP4 needs its outer scale
    assert rst(codes=f(0x10008)) == fq.FQ_ERR_ALIGN
    # calibration and selection
    assert L.fq_channel_absmax(f(), 64, 12, f(), None) == fq.FQ_ERR_SHAPE
    assert L.fq_channel_absmax(f(), 0, 64, f(), None) == fq.FQ_ERR_SHAPE
    assert L.fq_channel_absmax(f(), 64, 64, None, None) == fq.FQ_ERR_NULL
    assert L.fq_select_channels(f(), 64, 65, f(), f(), None) == fq.FQ_ERR_SHAPE
    assert L.fq_select_channels(f(), 64, -1, f(), f(), None) == fq.FQ_ERR_SHAPE
    assert L.fq_select_channels(f(), 60, 4, f(), f(), None) == fq.FQ_ERR_SHAPE
    assert L.fq_select_channels(f(), 64, 4, None, f(), None) == fq.FQ_ERR_NULL
    # retained-channel quantizer: either axis, every format
    mx, nvt = fq.fq_desc_mxfp4(), fq.fq_desc_nvfp4()
    col = fq.fq_desc_mxfp4(axis=fq.FQ_AXIS_COL)

    def fqr(d, retain=f(), scale=f(), rows=64, cols=64, y=f(), ws=f(), ws_bytes=4096):
        return L.fq_fake_quant_retain(ctypes.byref(d), f(), rows, cols, y, None, None, None,
                                      retain, scale, ws, ws_bytes, None)
    assert fqr(nvt, ws=None) == fq.FQ_ERR_NULL                  # per tensor: partial maxima
    assert fqr(nvt, ws_bytes=16) == fq.FQ_ERR_WORKSPACE
    assert fqr(col, rows=48) == fq.FQ_ERR_SHAPE                 # column groups of 32 rows
    assert fqr(mx, retain=None) == fq.FQ_ERR_NULL
    assert fqr(mx, scale=None) == fq.FQ_ERR_NULL
    assert fqr(mx, y=None) == fq.FQ_ERR_NULL
    assert fqr(mx, cols=48) == fq.FQ_ERR_SHAPE
    assert fqr(fq.fq_desc_nvfp4(outer=fq.FQ_OUTER_BLOCK128), cols=64) == fq.FQ_ERR_SHAPE
    assert fqr(fq.fq_desc_nvfp4(axis=fq.FQ_AXIS_COL), rows=64, cols=12) == fq.FQ_ERR_SHAPE
    # the retained linear: both masks required, K a multiple of 8
    nv, wcol = fq.fq_desc_nvfp4(), fq.fq_desc_nvfp4(axis=fq.FQ_AXIS_COL)
    big = 1 << 40
    assert L.fq_qlinear_fwd_retain(ctypes.byref(nv), ctypes.byref(wcol), f(), f(), 128, 128, 128,
                                   None, f(), f(), f(), big, None) == fq.FQ_ERR_NULL
    assert L.fq_qlinear_fwd_retain(ctypes.byref(nv), ctypes.byref(wcol), f(), f(), 128, 128, 128,
                                   f(), None, f(), f(), big, None) == fq.FQ_ERR_NULL
    g = fq.fq_desc_nvfp4(outer=fq.FQ_OUTER_BLOCK128, rounding=fq.FQ_ROUND_SR)
    assert L.fq_qlinear_bwd_retain(ctypes.byref(nv), ctypes.byref(wcol), ctypes.byref(g), f(),
                                   f(), f(), 128, 128, 128, None, f(), f(), f(), f(), big,
                                   None) == fq.FQ_ERR_NULL


def test_qlinear_bwd_validates(L):
    nv = fq.fq_desc_nvfp4()
    col = fq.fq_desc_nvfp4(axis=fq.FQ_AXIS_COL)
    g = fq.fq_desc_nvfp4(outer=fq.FQ_OUTER_BLOCK128, rounding=fq.FQ_ROUND_SR, seed=5)
    big = 1 << 40

    def call(dx_, dw_, dg_, M=128, K=128, N=128, ws_bytes=big, x=fake(), dy=fake(), rht=0):
        return L.fq_qlinear_bwd(ctypes.byref(dx_), ctypes.byref(dw_), ctypes.byref(dg_), rht, 7,
                                x, fake(), dy, M, K, N, fake(), fake(), fake(), ws_bytes, None)

    assert call(col, col, g) == fq.FQ_ERR_DESC                  # X must be blocked along K (rows)
    assert call(nv, nv, g) == fq.FQ_ERR_DESC                    # W must be blocked along K (cols)
    assert call(nv, col, g, M=64) == fq.FQ_ERR_SHAPE            # M not a multiple of 128 (g)
    assert call(nv, col, g, N=192) == fq.FQ_ERR_SHAPE           # N not a multiple of 128 (g)
    assert call(nv, col, nv, M=96) == fq.FQ_ERR_SHAPE           # M not a multiple of 64
    assert call(nv, col, g, K=120) == fq.FQ_ERR_SHAPE           # K not a multiple of 16
    assert call(nv, col, g, x=None) == fq.FQ_ERR_NULL
    assert call(nv, col, g, dy=fake(0x10004)) == fq.FQ_ERR_ALIGN
    assert call(nv, col, g, rht=32) == fq.FQ_ERR_DESC           # RHT blocks are 16 or 128
    assert call(nv, col, nv, M=192, N=192, rht=128) == fq.FQ_ERR_SHAPE   # M % 128
    need = L.fq_qlinear_bwd_workspace_size(ctypes.byref(nv), ctypes.byref(col), ctypes.byref(g),
                                           0, 128, 128, 128)
    assert need > 6 * 128 * 128 * 2
    assert call(nv, col, g, ws_bytes=need - 1) == fq.FQ_ERR_WORKSPACE
    # the double-block gradient quantizer rotates in registers: no extra space
    need_r = L.fq_qlinear_bwd_workspace_size(ctypes.byref(nv), ctypes.byref(col), ctypes.byref(g),
                                             128, 128, 128, 128)
    assert need_r == need
    # a per-tensor gradient quantizer needs the rotated operands materialized
    need_t = L.fq_qlinear_bwd_workspace_size(ctypes.byref(nv), ctypes.byref(col), ctypes.byref(nv),
                                             0, 128, 128, 128)
    need_tr = L.fq_qlinear_bwd_workspace_size(ctypes.byref(nv), ctypes.byref(col), ctypes.byref(nv),
                                              128, 128, 128, 128)
    assert need_tr >= need_t + 4 * 128 * 128 * 2
    assert call(nv, col, nv, ws_bytes=need_tr - 1, rht=128) == fq.FQ_ERR_WORKSPACE
    bad = fq.fq_desc_mxfp4()
    bad.reserved = 1
    assert L.fq_qlinear_bwd_workspace_size(ctypes.byref(nv), ctypes.byref(col), ctypes.byref(bad),
                                           0, 128, 128, 128) == 0


def test_hadamard_validates(L):
    x, y = fake(0x10000), fake(0x40000)
    assert L.fq_hadamard(x, 64, 96, fq.FQ_AXIS_ROW, 64, 1, y, None) == fq.FQ_ERR_DESC
    assert L.fq_hadamard(x, 64, 96, 2, 16, 1, y, None) == fq.FQ_ERR_DESC
    assert L.fq_hadamard(x, 64, 96, fq.FQ_AXIS_ROW, 128, 1, y, None) == fq.FQ_ERR_SHAPE
    assert L.fq_hadamard(x, 96, 64, fq.FQ_AXIS_COL, 128, 1, y, None) == fq.FQ_ERR_SHAPE
    assert L.fq_hadamard(x, 128, 12, fq.FQ_AXIS_COL, 16, 1, y, None) == fq.FQ_ERR_SHAPE
    assert L.fq_hadamard(None, 64, 128, fq.FQ_AXIS_ROW, 16, 1, y, None) == fq.FQ_ERR_NULL
    assert L.fq_hadamard(fake(0x10008), 64, 128, fq.FQ_AXIS_ROW, 16, 1, y, None) == fq.FQ_ERR_ALIGN
    assert L.fq_hadamard(x, 64, 128, fq.FQ_AXIS_ROW, 16, 1, fake(0x10100), None) == fq.FQ_ERR_SHAPE


def test_rotated_fake_quant_validates(L):
    mx = fq.fq_desc_mxfp4()
    nvt = fq.fq_desc_nvfp4()

    def call(d, rows=128, cols=128, blk=16, y=fake()):
        return L.fq_fake_quant_rht(ctypes.byref(d), fake(), rows, cols, blk, 3, y, None, None,
                                   None, None)
    assert call(nvt) == fq.FQ_ERR_DESC                  # per-tensor scale: not fused
    assert call(mx, blk=32) == fq.FQ_ERR_DESC
    assert call(mx, cols=96, blk=128) == fq.FQ_ERR_SHAPE
    assert call(mx, y=None) == fq.FQ_ERR_NULL
    col = fq.fq_desc_mxfp4(axis=fq.FQ_AXIS_COL)
    assert call(col, rows=96, blk=128) == fq.FQ_ERR_SHAPE


def test_status_strings(L):
    for s in range(7):
        assert L.fq_status_string(s).decode().startswith("FQ_")
    assert L.fq_version().decode().count(".") == 2


def test_binding_rejects_host_tensors():
    # the binding checks what the C library cannot see (device, layout, size)
    # before anything reaches a kernel
    import torch
    x = torch.zeros((4, 32), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        fq.fq_hadamard(x, 16)
