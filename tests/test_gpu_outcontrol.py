"""GPU parity of TetraJet-v2's OsciReset tracker and static outlier-channel
retention against the oracle: tracker state and reset weights bit-exact over
a multi-step trajectory; per-channel calibration maxima, the selected
channels and their FP8 scales bit-exact; the retained-channel fake quantizer
bit-exact (codes, scales, outer scales, y) on both formats and roundings,
including the 16384x4096 workload with 10 % of the channels retained."""
import numpy as np
import pytest
import torch

import fp4_block_quantization_fq_amd as fq
import oracle
import workloads as wl
from gpu_util import assert_product_bound, assert_same, make_desc, to_bits, to_dev, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


OSCI_CASES = [("mx", "row", (256, 512)), ("nv_tensor", "row", (128, 1024)),
              ("nv_128", "row", (96, 1024)), ("mx", "col", (512, 264)),
              ("nv_tensor", "col", (1024, 136)), ("nv_128", "col", (384, 200))]


def _gpu_quant(wbits, fmt, axis):
    """The GPU quantizer's fake quantization of the BF16 copy of w (checked
    against the oracle's), as the forward would produce q and its codes."""
    d = make_desc(fmt, "rne", axis)
    R, C = wbits.shape
    out = fq.alloc_outputs(d, R, C, DEV)
    y = fq.fq_fake_quant(d, to_dev(wbits), out=out)
    ref = oracle.fake_quant(wbits, fmt, "rne", axis)
    torch.cuda.synchronize()
    assert_same({"y": to_bits(y), "codes": to_np(out.codes), "scales": to_np(out.scales),
                 "outer": None if out.outer is None else to_np(out.outer)}, ref)
    return d, out, y, ref


@pytest.mark.parametrize("fmt,axis,shape", OSCI_CASES)
@pytest.mark.parametrize("target", ["centre", "grid"])
def test_osci_trajectory_matches_oracle(fmt, axis, shape, target):
    rng = np.random.default_rng(21)
    R, C = shape
    n = R * C
    w = (rng.standard_normal(n).astype(np.float32) * np.float32(0.02)).reshape(R, C)
    st_o = oracle.osci_state(n)
    st_g = fq.osci_state(n, DEV)
    tw = torch.from_numpy(w.copy()).to(DEV)
    for t in range(6):
        if t:
            w = (w + rng.standard_normal((R, C)).astype(np.float32) * np.float32(2e-4)).astype(np.float32)
            tw.copy_(torch.from_numpy(w))
        d, out, yq, ref = _gpu_quant(wl.f32_to_bf16_bits(w), fmt, axis)
        q = ref["y"].reshape(-1)
        oracle.osci_track(w.reshape(-1), q, st_o, first=(t == 0))
        fq.fq_osci_track(tw, yq, st_g, first=(t == 0))
        torch.cuda.synchronize()
        for k in ("w_prev", "dist_m", "dist_q"):
            assert np.array_equal(to_np(st_g[k]).view(np.uint32), st_o[k].view(np.uint32)), (t, k)
        assert np.array_equal(to_bits(st_g["q_prev"]), st_o["q_prev"]), t
    w_new, osc = oracle.osci_reset(w, q, st_o, 4.0, target, ref, fmt, axis)
    assert osc.any() and not osc.all()
    if target == "centre":
        fq.fq_osci_reset(tw, yq, st_g, 4.0, d, out, fq.FQ_OSCI_BIN_CENTRE)
        # the two readings part where the current code sits in the lopsided
        # bins of 2 and 4
        qv = oracle.bf16_bits_to_f64(q).astype(np.float32)
        assert (w_new[osc] != qv[osc]).any()
    else:
        fq.fq_osci_reset(tw, yq, st_g, 4.0, target=fq.FQ_OSCI_GRID_VALUE)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(tw).reshape(-1).view(np.uint32), w_new.view(np.uint32))
    for k in ("w_prev", "dist_m", "dist_q"):
        assert np.array_equal(to_np(st_g[k]).view(np.uint32), st_o[k].view(np.uint32)), k


@pytest.mark.parametrize("shape", [(1000, 4104), (64, 64)])
def test_channel_selection_matches_oracle(shape):
    R, C = shape
    x, cols = wl.activation_and_outlier_channels(shape, 1.0, 8, 100.0, seed=R)
    half = R // 2
    am_o = oracle.channel_absmax(x[half:], oracle.channel_absmax(x[:half]))
    tx = to_dev(x)
    am_g = fq.fq_channel_absmax(tx[:half].contiguous())
    fq.fq_channel_absmax(tx[half:].contiguous(), am_g)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(am_g).view(np.uint32), am_o)
    for k in (0, 8, C // 10, C):
        ret_o, sc_o = oracle.select_channels(am_o, k)
        ret_g, sc_g = fq.fq_select_channels(am_g, k)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(ret_g), np.packbits(ret_o, bitorder="little")), k
        assert np.array_equal(to_np(sc_g).view(np.uint32), sc_o.view(np.uint32)), k
        if k == 8:
            assert np.flatnonzero(ret_o).tolist() == cols.tolist()


def _retain_case(x, fmt, rnd, k, seed=31, axis="row"):
    ret_o, sc_o = oracle.select_channels(oracle.channel_absmax(x), k)
    ref = oracle.fake_quant_retained(x, fmt, ret_o, sc_o, rnd, axis, seed)
    d = make_desc(fmt, rnd, axis, seed)
    tx = to_dev(x)
    R, C = x.shape
    out = fq.alloc_outputs(d, R, C, tx.device)
    retain = torch.from_numpy(np.packbits(ret_o, bitorder="little")).to(DEV)
    y = fq.fq_fake_quant_retain(d, tx, retain, torch.from_numpy(sc_o).to(DEV), out=out)
    torch.cuda.synchronize()
    got = {"y": to_bits(y), "codes": to_np(out.codes), "scales": to_np(out.scales),
           "outer": None if out.outer is None else to_np(out.outer)}
    assert_same(got, ref, tag=f"retain {fmt}/{rnd}/{axis}/{x.shape}/k={k}")


@pytest.mark.parametrize("shape", [(256, 384), (384, 1024)])
@pytest.mark.parametrize("rnd", ["rne", "sr"])
@pytest.mark.parametrize("fmt", ["mx", "nv_128", "nv_tensor"])
@pytest.mark.parametrize("axis", ["row", "col"])
def test_fake_quant_retain_matches_oracle(fmt, rnd, shape, axis):
    x = wl.activation_with_outlier_channels(shape, 1.0, 6, 100.0, seed=shape[0])
    for k in (0, 6, shape[1] // 10):
        _retain_case(x, fmt, rnd, k, axis=axis)


def test_fake_quant_retain_ragged_rows():
    # 130 rows: a partial row group (row axis); column tiles of 256 rows with
    # a ragged end (column axis needs rows in whole blocks: 160)
    x = wl.activation_with_outlier_channels((130, 1024), 1.0, 6, 100.0, seed=130)
    for fmt in ("mx", "nv_128", "nv_tensor"):
        _retain_case(x, fmt, "sr", 102)
    x = wl.activation_with_outlier_channels((160, 1032), 1.0, 6, 100.0, seed=160)
    for fmt in ("mx", "nv_tensor"):
        _retain_case(x, fmt, "sr", 103, axis="col")


@pytest.mark.parametrize("fmt,axis", [("mx", "row"), ("nv_tensor", "row"), ("nv_128", "col"),
                                      ("mx", "col")])
def test_fake_quant_retain_every_bf16_value(fmt, axis):
    """Every finite BF16 value through the FP8 channel path: all 64 columns
    retained, each column holding the values whose pattern is its index mod
    64 (every exponent), under 64 channel scales from 2^-40 to 2^30 (plus 1,
    1/3 and 0), rotated over three calls so that every value meets three
    scales; bit for bit against the oracle (y, and the empty FP4 part)."""
    pats = np.arange(65536, dtype=np.uint32)
    finite = pats[(pats & 0x7F80) != 0x7F80].astype(np.uint16)
    x = np.zeros(1024 * 64, np.uint16)
    x[:finite.size] = finite
    x = x.reshape(1024, 64)
    base = (2.0 ** np.linspace(-40, 30, 64)).astype(np.float32) * np.float32(1.37)
    base[0], base[1], base[2] = 1.0, np.float32(1.0 / 3.0), 0.0
    ret = np.ones(64, np.uint8)
    retain = torch.from_numpy(np.packbits(ret, bitorder="little")).to(DEV)
    d = make_desc(fmt, "rne", axis)
    tx = to_dev(x)
    for shift in (0, 21, 42):
        sc = np.roll(base, shift).astype(np.float32)
        ref = oracle.fake_quant_retained(x, fmt, ret, sc, "rne", axis, 0)
        out = fq.alloc_outputs(d, 1024, 64, tx.device)
        y = fq.fq_fake_quant_retain(d, tx, retain, torch.from_numpy(sc).to(DEV), out=out)
        torch.cuda.synchronize()
        got = {"y": to_bits(y), "codes": to_np(out.codes), "scales": to_np(out.scales),
               "outer": None if out.outer is None else to_np(out.outer)}
        assert_same(got, ref, tag=f"every BF16 value, {fmt}/{axis}, scale shift {shift}")


def test_fake_quant_retain_full_size():
    x = wl.nv_activation(16384, 4096, seed=3)
    _retain_case(x, "nv_128", "sr", 410, seed=1234)
    _retain_case(x, "nv_128", "sr", 410, seed=1234, axis="col")
    _retain_case(x, "nv_tensor", "rne", 410, axis="row")


def _linear_retained(M, K, N, fmts, frac=0.1, seed_g=1234):
    """The retained linear forward and backward against the oracle's
    composition: X_hat bit for bit, every product element within the
    FP32-accumulation / BF16-rounding bound, dropped STE entries exactly 0."""
    fx, fw, fg = fmts
    x, _ = wl.activation_and_outlier_channels((M, K), 1.0, 8, 100.0, seed=61)
    w = wl.normal_bf16((K, N), 0.02, 62)
    dy = wl.normal_bf16((M, N), 1e-3, 63)
    k = max(1, int(round(frac * K)))
    ret_o, sc_o = oracle.select_channels(oracle.channel_absmax(x), k)
    retain = torch.from_numpy(np.packbits(ret_o, bitorder="little")).to(DEV)
    cs = torch.from_numpy(sc_o).to(DEV)
    dx_, dw_, dg_ = make_desc(fx, "rne", "row"), make_desc(fw, "rne", "col"), \
        make_desc(fg, "sr", "row", seed_g)
    xd, wd, dyd = to_dev(x), to_dev(w), to_dev(dy)
    ws = fq.qlinear_workspace(dx_, dw_, M, K, N, xd.device)
    y = fq.fq_qlinear_fwd_retain(dx_, dw_, xd, wd, retain, cs, ws=ws)
    gx, gw = fq.fq_qlinear_bwd_retain(dx_, dw_, dg_, xd, wd, dyd, retain, cs)
    torch.cuda.synchronize()
    ref = oracle.qlinear(x, w, fx, fw, retain=ret_o, chan_scale=sc_o)
    xhat, _ = fq.qlinear_workspace_views(ws, M, K, N)
    assert np.array_equal(to_bits(xhat), ref["xhat"]), "X_hat with retained channels"
    f64 = oracle.bf16_bits_to_f64
    absprod = np.abs(f64(ref["xhat"])) @ np.abs(f64(ref["what"]))
    assert_product_bound(f64(to_bits(y)), ref["y"], absprod, K, tag="retained forward")
    rb = oracle.qlinear_bwd(x, w, dy, fx, fw, fg, "sr", seed_g, retain=ret_o, chan_scale=sc_o)
    for name, got, keep, a, b, kdim in (
            ("dx", gx, rb["keep_x"], f64(rb["q_dy_n"]), f64(rb["q_w_n"]).T, N),
            ("dw", gw, rb["keep_w"], f64(rb["q_x_m"]).T, f64(rb["q_dy_m"]), M)):
        g = f64(to_bits(got))
        assert_product_bound(g, a @ b, np.abs(a) @ np.abs(b), kdim, keep=keep,
                             tag=f"retained backward {name}")


@pytest.mark.parametrize("fmts", [("nv_tensor", "nv_tensor", "nv_128"), ("mx", "mx", "mx"),
                                  ("nv_128", "nv_tensor", "nv_tensor")])
def test_linear_retained_small(fmts):
    _linear_retained(256, 384, 256, fmts)


def test_linear_retained_full_size():
    _linear_retained(8192, 2880, 5760, ("nv_tensor", "nv_tensor", "nv_128"))


@pytest.mark.parametrize("shape,fmt", [((1, 4), None), ((1, 132), None),
                                       ((33, 4096 + 4), None), ((33, 4128), "mx"),
                                       ((3, 4096 * 11), "nv_128")])
def test_osci_sizes(shape, fmt):
    # the smallest size, a size that leaves a partial wave, and ones that
    # leave a partial workgroup: every element tracked and checked (the
    # grid-value target where the shape cannot be blocked)
    R, C = shape
    n = R * C
    rng = np.random.default_rng(n)
    w0 = rng.standard_normal((R, C)).astype(np.float32)
    w1 = (w0 + rng.standard_normal((R, C)).astype(np.float32) * np.float32(1e-3)).astype(np.float32)
    if fmt is None:
        q0 = wl.f32_to_bf16_bits(w0)
        q1 = wl.f32_to_bf16_bits(np.where(rng.random((R, C)) < 0.5, w1, w0 + np.float32(0.25)))
        tq0, tq1 = to_dev(q0), to_dev(q1)
    else:
        _, _, tq0, r0 = _gpu_quant(wl.f32_to_bf16_bits(w0), fmt, "row")
        d, out, tq1, r1 = _gpu_quant(wl.f32_to_bf16_bits(w1), fmt, "row")
        q0, q1 = r0["y"], r1["y"]
    st_o, st_g = oracle.osci_state(n), fq.osci_state(n, DEV)
    tw = torch.from_numpy(w0.copy()).to(DEV)
    oracle.osci_track(w0.reshape(-1), q0.reshape(-1), st_o, first=True)
    fq.fq_osci_track(tw, tq0, st_g, first=True)
    tw.copy_(torch.from_numpy(w1))
    oracle.osci_track(w1.reshape(-1), q1.reshape(-1), st_o, first=False)
    fq.fq_osci_track(tw, tq1, st_g)
    if fmt is None:
        w_new, osc = oracle.osci_reset(w1, q1, st_o, 8.0, "grid")
        fq.fq_osci_reset(tw, tq1, st_g, 8.0, target=fq.FQ_OSCI_GRID_VALUE)
    else:
        w_new, osc = oracle.osci_reset(w1, q1, st_o, 0.5, "centre", r1, fmt, "row")
        fq.fq_osci_reset(tw, tq1, st_g, 0.5, d, out)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(tw).reshape(-1).view(np.uint32), w_new.view(np.uint32))
    assert np.array_equal(to_bits(st_g["q_prev"]).reshape(-1), st_o["q_prev"])
