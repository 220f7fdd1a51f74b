"""Pins of the oracle's OsciReset tracker and of the static outlier-channel
retention ("Resumo Tecnico: TetraJet-v2", sec. 2.B and 2.C): hand-computed
trajectories with exactly representable steps, the retained channels found
by the workload generator's own choice, the FP8 encoding checked against
torch's float8_e4m3fn cast, and the FP4 part checked against the plain
quantizer on the same tensor with the retained columns zeroed."""
import numpy as np
import pytest
import torch

import oracle
from workloads import activation_and_outlier_channels, f32_to_bf16_bits


def bf(vals):
    return f32_to_bf16_bits(np.asarray(vals, np.float32))


def run_traj(ws, qs, tau):
    st = oracle.osci_state(len(ws[0]))
    for t, (w, q) in enumerate(zip(ws, qs)):
        oracle.osci_track(np.asarray(w, np.float32), bf(q), st, first=(t == 0))
    dm, dq = st["dist_m"].copy(), st["dist_q"].copy()
    w_new, osc = oracle.osci_reset(np.asarray(ws[-1], np.float32), bf(qs[-1]), st, tau)
    return dm, dq, w_new, osc, st


def test_osci_steady_weight_is_not_reset():
    # the master weight walks up by 1/8 per step; its quantized value moves
    # once (1.0 -> 1.5): dist_m = 3/8, dist_q = 1/2, risk 4/3 < 2
    ws = [[1.0], [1.125], [1.25], [1.375]]
    qs = [[1.0], [1.0], [1.0], [1.5]]
    dm, dq, w_new, osc, _ = run_traj(ws, qs, 2.0)
    assert dm.tolist() == [0.375] and dq.tolist() == [0.5]
    assert not osc[0] and w_new.tolist() == [1.375]


def test_osci_flipping_weight_is_reset_to_its_quantized_value():
    # the master weight hops across the 1.0 / 1.5 boundary (1.25) by 1/32,
    # the quantized value flips every step: dist_m = 3/32, dist_q = 3/2
    ws = [[1.234375], [1.265625], [1.234375], [1.265625]]
    qs = [[1.0], [1.5], [1.0], [1.5]]
    dm, dq, w_new, osc, st = run_traj(ws, qs, 2.0)
    assert dm.tolist() == [0.09375] and dq.tolist() == [1.5]
    assert osc[0] and w_new.tolist() == [1.5]
    # a new window starts from the reset weight
    assert st["dist_m"].tolist() == [0.0] and st["dist_q"].tolist() == [0.0]
    assert st["w_prev"].tolist() == [1.5]


def test_osci_degenerate_windows():
    # element 0: master still, quantized value moved -> reset; element 1:
    # nothing moved -> kept; element 2: risk exactly tau -> kept (strict >)
    ws = [[2.0, 3.0, 1.0], [2.0, 3.0, 1.5]]
    qs = [[2.0, 3.0, 1.0], [3.0, 3.0, 2.0]]
    dm, dq, w_new, osc, _ = run_traj(ws, qs, 2.0)
    assert dm.tolist() == [0.0, 0.0, 0.5] and dq.tolist() == [1.0, 0.0, 1.0]
    assert osc.tolist() == [True, False, False]
    assert w_new.tolist() == [3.0, 3.0, 1.5]


def test_selection_finds_the_generated_outlier_channels():
    x, cols = activation_and_outlier_channels((512, 384), 1.0, 8, 100.0, seed=12)
    amax = oracle.channel_absmax(x[:256])
    amax = oracle.channel_absmax(x[256:], amax)          # two calibration batches
    retain, scale = oracle.select_channels(amax, 8)
    assert np.flatnonzero(retain).tolist() == cols.tolist()
    assert np.all(scale[~retain] == 0)


def test_selection_scale_and_ties():
    a = bf([448.0, 1.75, 1.75, 0.5]).astype(np.uint32)
    retain, scale = oracle.select_channels(a, 2)
    assert retain.tolist() == [True, True, False, False]      # tie: lower index first
    assert scale.tolist() == [1.0, 0.00390625, 0.0, 0.0]      # 448/448, 1.75/448 = 2^-8


@pytest.mark.parametrize("fmt", ["mx", "nv_128"])
@pytest.mark.parametrize("rnd", ["rne", "sr"])
def test_retain_nothing_is_plain_fake_quant(fmt, rnd):
    x, _ = activation_and_outlier_channels((64, 256), 1.0, 4, 100.0, seed=13)
    C = x.shape[1]
    r = oracle.fake_quant_retain(x, fmt, np.zeros(C, bool), np.zeros(C, np.float32), rnd, 5)
    p = oracle.fake_quant(x, fmt, rnd, "row", 5)
    for k in ("codes", "scales", "outer", "y"):
        if p[k] is None:
            assert r[k] is None
        else:
            assert np.array_equal(r[k], p[k]), k


@pytest.mark.parametrize("fmt", ["mx", "nv_128"])
def test_retained_columns_leave_the_fp4_blocks(fmt):
    # the FP4 part equals the plain quantizer on the tensor whose retained
    # columns are zero: they take no part in any block or outer maximum
    x, cols = activation_and_outlier_channels((64, 256), 1.0, 4, 100.0, seed=14)
    C = x.shape[1]
    amax = oracle.channel_absmax(x)
    retain, scale = oracle.select_channels(amax, 4)
    assert np.flatnonzero(retain).tolist() == cols.tolist()
    r = oracle.fake_quant_retain(x, fmt, retain, scale, "sr", 7)
    xz = x.copy()
    xz[:, retain] = 0
    p = oracle.fake_quant(xz, fmt, "sr", "row", 7)
    assert np.array_equal(r["scales"], p["scales"])
    if fmt == "nv_128":
        assert np.array_equal(r["outer"], p["outer"])
    assert np.array_equal(r["codes"], p["codes"])            # retained positions: code 0
    assert np.array_equal(r["y"][:, ~retain], p["y"][:, ~retain])


def test_retained_columns_are_fp8_e4m3():
    x, cols = activation_and_outlier_channels((64, 256), 1.0, 4, 100.0, seed=15)
    amax = oracle.channel_absmax(x)
    retain, scale = oracle.select_channels(amax, 4)
    r = oracle.fake_quant_retain(x, "mx", retain, scale)
    xf = oracle.bf16_bits_to_f64(x).astype(np.float32)
    for c in np.flatnonzero(retain):
        a = np.abs(xf[:, c]) / scale[c]                     # FP32 quotient
        assert a.max() < 464.0                               # inside torch's rounding range
        e = torch.from_numpy(a).to(torch.float8_e4m3fn).to(torch.float32).numpy()
        mag = (e * scale[c]).astype(np.float32)
        want = f32_to_bf16_bits(np.where(np.signbit(xf[:, c]), -mag, mag))
        assert np.array_equal(r["y"][:, c], want), c
