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
    """Detection on hand trajectories; the reset goes to the quantized value
    (the "grid" target), which equals the bin centre at the grid points these
    trajectories use (0, 0.5, 1, 1.5 and 3 have symmetric bins)."""
    st = oracle.osci_state(len(ws[0]))
    for t, (w, q) in enumerate(zip(ws, qs)):
        oracle.osci_track(np.asarray(w, np.float32), bf(q), st, first=(t == 0))
    dm, dq = st["dist_m"].copy(), st["dist_q"].copy()
    w_new, osc = oracle.osci_reset(np.asarray(ws[-1], np.float32), bf(qs[-1]), st, tau,
                                   target="grid")
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


def test_bin_centres_by_hand():
    # E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; round-to-nearest bins
    # [-.25, .25], [.25, .75], [.75, 1.25], [1.25, 1.75], [1.75, 2.5],
    # [2.5, 3.5], [3.5, 5], [5, 7] (the last one by the reading)
    assert oracle.e2m1_bin_centres() == [0.0, 0.5, 1.0, 1.5, 2.125, 3.0, 4.25, 6.0]


def test_bin_centres_lie_in_their_rounding_bins():
    # every centre rounds to its own code, and so does every point of the bin
    # short of its two ends (the oracle's RNE is pinned on its own)
    c = oracle.e2m1_bin_centres()
    g = list(oracle.E2M1_GRID)
    for m in range(8):
        assert oracle.e2m1_rne(c[m]) == m
        hi = (g[m] + g[m + 1]) / 2 if m < 7 else 7.0
        lo = (g[m - 1] + g[m]) / 2 if m else 0.0
        for t in np.linspace(lo, hi, 33)[1:-1]:
            assert oracle.e2m1_rne(float(t)) == m, (m, t)
        assert c[m] - lo == hi - c[m] or m == 0


def _osci_case(rows_of_w, fmt, tau, axis="row"):
    """Track a trajectory of [R, C] master weights quantized with fmt (RNE)
    along axis, then reset with both targets.  Returns the two new weights."""
    st_c = oracle.osci_state(rows_of_w[0].size)
    st_g = oracle.osci_state(rows_of_w[0].size)
    for t, w in enumerate(rows_of_w):
        q = oracle.fake_quant(bf(w), fmt, "rne", axis)
        for st in (st_c, st_g):
            oracle.osci_track(np.asarray(w, np.float32).reshape(-1), q["y"].reshape(-1), st,
                              first=(t == 0))
    w = np.asarray(rows_of_w[-1], np.float32)
    wc, osc_c = oracle.osci_reset(w, q["y"], st_c, tau, "centre", q, fmt, axis)
    wg, osc_g = oracle.osci_reset(w, q["y"], st_g, tau, "grid")
    assert np.array_equal(osc_c, osc_g)
    return wc.reshape(w.shape), wg.reshape(w.shape), osc_c.reshape(w.shape)


def test_osci_reset_to_bin_centre_mxfp4():
    # one 32-block with amax 0.75 -> E8M0 scale 2^-3.  Element 1 hops across
    # the 1.5 / 2 boundary (1.75 * 2^-3 = 0.21875): a = 1.8125, 1.6875, 1.8125
    # -> q = 0.25, 0.1875, 0.25; element 2 across the 3 / 4 boundary
    # (-0.4375): a = 3.5625, 3.4375, 3.5625 -> q = -0.5, -0.375, -0.5.
    # dist_m = 1/32 for both; dist_q = 1/8 and 1/4: risks 4 and 8 > 2.
    # Current codes 4 (2.0) and 0xE (-4.0): bin centres 2.125 * 2^-3 = 0.265625
    # and -4.25 * 2^-3 = -0.53125; the grid target gives 0.25 and -0.5.
    base = np.zeros((1, 32), np.float32)
    base[0, 0] = 0.75
    traj = []
    for w1, w2 in ((0.2265625, -0.4453125), (0.2109375, -0.4296875), (0.2265625, -0.4453125)):
        b = base.copy()
        b[0, 1], b[0, 2] = w1, w2
        traj.append(b)
    wc, wg, osc = _osci_case(traj, "mx", 2.0)
    assert np.flatnonzero(osc).tolist() == [1, 2]
    assert wc[0, :3].tolist() == [0.75, 0.265625, -0.53125]
    assert wg[0, :3].tolist() == [0.75, 0.25, -0.5]


def test_osci_reset_to_bin_centre_nvfp4():
    # NVFP4 per tensor, one 16-block with amax 2.625: s_t = 2^-10, block scale
    # 448, s_eff = 0.4375.  Element 1: 0.78125, 0.75, 0.78125 -> a = 1.7857.. /
    # 1.7142.. -> codes 4, 3, 4 (q = 0.875, 0.65625, 0.875); dist_m = 1/16,
    # dist_q = 7/16 (risk 7).  Element 2: -1.65625, -1.5, -1.65625 -> a =
    # 3.7857.. / 3.4285.. -> codes 0xE, 0xD (q = -1.75, -1.3125); dist_m =
    # 5/16, dist_q = 7/8 (risk 2.8).  Centres: 2.125 * 0.4375 = 0.9296875 and
    # -4.25 * 0.4375 = -1.859375; grid values 0.875 and -1.75.
    base = np.zeros((1, 16), np.float32)
    base[0, 0] = 2.625
    traj = []
    for w1, w2 in ((0.78125, -1.65625), (0.75, -1.5), (0.78125, -1.65625)):
        b = base.copy()
        b[0, 1], b[0, 2] = w1, w2
        traj.append(b)
    wc, wg, osc = _osci_case(traj, "nv_tensor", 2.0)
    assert np.flatnonzero(osc).tolist() == [1, 2]
    assert wc[0, :3].tolist() == [2.625, 0.9296875, -1.859375]
    assert wg[0, :3].tolist() == [2.625, 0.875, -1.75]


def test_osci_reset_centre_column_layout():
    # W [32, 8] grouped down its columns (MXFP4): column 3 has amax 0.75
    # (scale 2^-3), the others amax 48 (scale 2^3).  Element (5, 3) flips
    # between codes 3 and 4 of its column's scale and is reset to
    # 2.125 * 2^-3; read in the row layout its code and scale would differ.
    base = np.zeros((32, 8), np.float32)
    base[0, :] = 48.0
    base[0, 3] = 0.75
    traj = []
    for v in (0.2265625, 0.2109375, 0.2265625):
        b = base.copy()
        b[5, 3] = v
        traj.append(b)
    wc, wg, osc = _osci_case(traj, "mx", 2.0, axis="col")
    assert np.argwhere(osc).tolist() == [[5, 3]]
    assert wc[5, 3] == 0.265625 and wg[5, 3] == 0.25
    assert np.array_equal(np.delete(wc.reshape(-1), 5 * 8 + 3), np.delete(traj[-1].reshape(-1), 5 * 8 + 3))


def test_bin_centre_values_signed_zero_and_top_bin():
    # code 8 (-0) -> -0.0; code 7 (6) -> 6 * s; code 0xF -> -6 * s
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 6.5          # a = 6.5 -> clipped, code 7, scale 1 (amax 6.5 -> 2^0)
    x[0, 1] = -0.125       # a = 0.125 -> code 8
    x[0, 2] = -5.5         # code 0xF
    q = oracle.fake_quant(bf(x), "mx")
    v = oracle.bin_centre_values(q["codes"], q["scales"], q["outer"], "mx", (1, 32))
    assert v[0, :3].tolist() == [6.0, 0.0, -6.0]
    assert np.signbit(v[0, 1])


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


# ---------------------------------------------------------------------------
# retention on both axes, every format, and in the linear (sec. 2.C: the
# retained channels stay FP8 in the forward and the backward pass)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", ["mx", "nv_128"])
@pytest.mark.parametrize("rnd", ["rne", "sr"])
def test_retained_composition_equals_the_loop_oracle_on_rows(fmt, rnd):
    # the zero-and-overlay composition against the C loop that masks the
    # retained columns out of each block (two formulations of one reading)
    x, cols = activation_and_outlier_channels((64, 384), 1.0, 8, 100.0, seed=3)
    retain = np.zeros(384, bool)
    retain[cols] = True
    retain[[5, 6, 200]] = True
    scale = np.where(retain, np.float32(0.37), np.float32(0)).astype(np.float32)
    a = oracle.fake_quant_retained(x, fmt, retain, scale, rnd, "row", 99)
    b = oracle.fake_quant_retain(x, fmt, retain, scale, rnd, 99)
    for k in ("codes", "scales", "outer", "y"):
        if a[k] is None:
            assert b[k] is None
            continue
        assert np.array_equal(a[k], b[k]), k


def test_fp8_clip_rule_by_hand():
    # scale 1: |x| = 448 is kept, 464 (rounds to 448) and 480 are clipped;
    # scale 0.5: 224 -> a = 448 kept, 232 -> a = 464 clipped; scale 0: kept, +-0
    x = bf([448.0, 464.0, -480.0, 224.0, 232.0, -3.0, 1.0])
    s = np.array([1, 1, 1, 0.5, 0.5, 0, 1], np.float32)
    y, clip = oracle.fp8_fake(x, s)
    assert clip.tolist() == [0, 1, 1, 0, 1, 0, 0]
    assert f32(y).tolist() == [448.0, 448.0, -448.0, 224.0, 224.0, -0.0, 1.0]
    assert np.signbit(f32(y)[5])


def f32(bits):
    return oracle.bf16_bits_to_f64(bits).astype(np.float32)


def test_column_axis_retention_by_hand():
    # x [32, 8], MXFP4 along rows of each column (32-row blocks).  Column 3 is
    # retained with scale 2^-6: its values are FP8 of x / 2^-6 (1.3 -> 83.2
    # -> E4M3 80 -> 1.25; 0.1 -> 6.4 -> 6.5 -> 0.1015625), it has FP4 codes 0
    # and the E8M0 code of an empty block (0).  Column 0 keeps its FP4 block:
    # amax 6 -> scale 1, 1.3 -> 1.5 (RNE).
    x = np.zeros((32, 8), np.float32)
    x[0, 0], x[1, 0] = 6.0, 1.3
    x[0, 3], x[1, 3] = 1.3, -0.1
    xb = bf(x)
    retain = np.zeros(8, bool)
    retain[3] = True
    scale = np.zeros(8, np.float32)
    scale[3] = 2.0 ** -6
    r = oracle.fake_quant_retained(xb, "mx", retain, scale, "rne", "col")
    y = f32(r["y"])
    assert y[0, 3] == 1.25 and y[1, 3] == -0.1015625
    assert y[0, 0] == 6.0 and y[1, 0] == 1.5
    assert r["scales"][3].tolist() == [0]                    # column 3's only block: empty
    assert r["scales"][0].tolist() == [127]
    assert np.all(r["codes"][3] == 0)
    assert r["clip"].sum() == 0


def test_per_tensor_retention_leaves_the_retained_maximum_out():
    # NVFP4 per tensor: the retained channel holds the largest value (100);
    # the tensor scale comes from the others' maximum 2.625 = 2688 * 2^-10
    # (block scale 448 * 2^-10 = 0.4375 for the block of 2.625: a = 6 and 1;
    # 0.4375 sits in that block along rows at (0, 2), along columns at (1, 1))
    x = np.zeros((16, 16), np.float32)
    x[:, 0] = 100.0
    x[0, 1] = 2.625
    x[0, 2] = 0.4375
    x[1, 1] = 0.4375
    xb = bf(x)
    retain = np.zeros(16, bool)
    retain[0] = True
    scale = np.zeros(16, np.float32)
    scale[0] = np.float32(100.0 / 448.0)
    for axis, at in (("row", (0, 2)), ("col", (1, 1))):
        r = oracle.fake_quant_retained(xb, "nv_tensor", retain, scale, "rne", axis)
        assert r["outer"].tolist() == [2.0 ** -10], axis
        y = f32(r["y"])
        assert y[0, 1] == 2.625 and y[at] == 0.4375, axis
        assert y[0, 0] == 100.0, axis                         # 448 * s, s = 100/448


def _fp8_exact_operands(M, K, N, seed):
    """MXFP4 grid operands (every 32-block along both axes has a 6, scale 1),
    X's retained channels holding E4M3 multiples of their scale 2^-6 that the
    E2M1 grid does not hold (1.25, 2.5, 3.5, ...), so FP8 keeps them exactly
    and FP4 would not."""
    GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    rng = np.random.default_rng(seed)

    def grid(R, C):
        v = rng.choice(GRID, size=(R, C)) * rng.choice([-1.0, 1.0], size=(R, C))
        i, j = np.indices((R, C))
        v[(i + j) % 32 == 0] = 6.0
        return v
    x, w, dy = grid(M, K), grid(K, N), grid(M, N)
    retain = np.zeros(K, bool)
    retain[rng.choice(K, size=K // 10, replace=False)] = True
    FP8_ONLY = np.array([1.25, 2.5, 3.5, 5.0, 0.75, 1.75])
    x[:, retain] = rng.choice(FP8_ONLY, size=(M, int(retain.sum()))) * \
        rng.choice([-1.0, 1.0], size=(M, int(retain.sum())))
    scale = np.where(retain, np.float32(2.0 ** -6), np.float32(0)).astype(np.float32)
    return x, w, dy, retain, scale


def test_linear_with_retained_channels_exact():
    M, K, N = 64, 160, 96
    x, w, dy, retain, scale = _fp8_exact_operands(M, K, N, 5)
    xb, wb, gb = bf(x), bf(w), bf(dy)
    r = oracle.qlinear(xb, wb, "mx", "mx", retain=retain, chan_scale=scale)
    assert np.array_equal(oracle.bf16_bits_to_f64(r["xhat"]), x)       # FP8 kept them
    assert np.array_equal(r["y"], x @ w)
    # without retention the same channels would be rounded to the E2M1 grid
    plain = oracle.qlinear(xb, wb, "mx", "mx")
    assert not np.array_equal(oracle.bf16_bits_to_f64(plain["xhat"]), x)
    b = oracle.qlinear_bwd(xb, wb, gb, "mx", "mx", "mx", "sr", 11, retain=retain,
                           chan_scale=scale)
    assert np.array_equal(b["keep_x"], np.ones_like(x))
    assert np.array_equal(b["dx"], dy @ w.T)
    assert np.array_equal(b["dw"], x.T @ dy)                           # X_hat along M: FP8 too
    bp = oracle.qlinear_bwd(xb, wb, gb, "mx", "mx", "mx", "sr", 11)
    assert not np.array_equal(bp["dw"], x.T @ dy)
