"""Hand-worked blocks: expected codes, scales and values derived by hand from
the format definitions (E2M1 grid, E8M0 rule floor(log2 amax) - 2, NVFP4
two-level scale amax / (6 * 448) with an E4M3 block scale), written next to
each case.  None of these numbers come from the oracle or the GPU library."""
import numpy as np

import oracle
from workloads import f32_to_bf16_bits


def bf(vals):
    return f32_to_bf16_bits(np.asarray(vals, np.float32))


def f32(bits):
    return oracle.bf16_bits_to_f64(bits).astype(np.float32)


def unpack(codes):
    codes = np.asarray(codes, np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = codes & 15
    out[..., 1::2] = codes >> 4
    return out


def test_mx_worked_block():
    # amax 7 -> floor(log2 7) = 2 -> k = 0 -> E8M0 code 127, scale 1
    x = [1, -0.30078125, 5.5, 0.25, -2.5, 0.75, 3.5, -7, 1.25, -1.75, 5] + [0] * 21
    r = oracle.fake_quant(bf([x]), "mx")
    assert r["scales"].tolist() == [[127]]
    want_codes = [0x2, 0x9, 0x7, 0x0, 0xC, 0x2, 0x6, 0xF, 0x2, 0xC, 0x6] + [0] * 21
    assert unpack(r["codes"])[0].tolist() == want_codes
    assert r["codes"][0, :6].tolist() == [0x92, 0x07, 0x2C, 0xF6, 0xC2, 0x06]
    want_y = [1, -0.5, 6, 0, -2, 1, 4, -6, 1, -2, 4] + [0] * 21
    assert f32(r["y"])[0].tolist() == want_y
    # only -7 (a = 7 > 6) is clipped
    assert np.flatnonzero(r["clip"][0]).tolist() == [7]


def test_mx_clamped_block_max():
    # amax 0.10009765625 = 1.6015625 * 2^-4 -> k = -6 -> code 121, s = 2^-6;
    # a = 6.40625 saturates to 6 (code 7) and is clipped;
    # -0.0234375 / 2^-6 = -1.5 -> code 0xB, not clipped
    x = [0.10009765625, -0.0234375] + [0] * 30
    r = oracle.fake_quant(bf([x]), "mx")
    assert r["scales"].tolist() == [[121]]
    assert unpack(r["codes"])[0, :2].tolist() == [0x7, 0xB]
    y = f32(r["y"])[0]
    assert y[0] == 6 * 2.0 ** -6
    assert y[1] == -1.5 * 2.0 ** -6
    assert r["clip"][0, 0] == 1 and r["clip"][0, 1] == 0


def test_mx_subnormal_block_clamps_scale():
    # BF16 subnormals.  Block 1: amax = 3 * 2^-133 -> floor(log2) = -132 ->
    # k = -134 clamps to -127 (code 0); a = 3 * 2^-133 * 2^127 = 0.046875 -> 0.
    x = np.zeros((1, 64), np.uint16)
    x[0, 0] = 0x0003          # 3 * 2^-133
    x[0, 32] = 0x0040         # 2^-127 (bf16 subnormal, 0x40 * 2^-133)
    x[0, 33] = 0x0060         # 1.5 * 2^-127
    r = oracle.fake_quant(x, "mx")
    assert r["scales"].tolist() == [[0, 0]]
    c = unpack(r["codes"])[0]
    # block 2: amax 1.5 * 2^-127 -> floor(log2) = -127 -> k = -129 -> clamps
    # to -127; a = 1 and 1.5 -> codes 2 and 3, exact y
    assert c[0] == 0 and c[32] == 2 and c[33] == 3
    assert r["y"][0, 32] == 0x0040 and r["y"][0, 33] == 0x0060


def _nv_tensor_example():
    # Tensor absmax A = 2.625 -> s_t = 2.625 / 2688 = 2^-10 exactly.
    b1 = [2.625, 0.4375, -0.65625, 0.109375, 1.53125, 2.1875] + [0] * 10
    b2 = [0.1875, 0.046875, -0.0078125] + [0] * 13
    b3 = [1.34375, 0.5] + [0] * 14
    return bf([b1 + b2 + b3])


def test_nv_tensor_worked_blocks():
    r = oracle.fake_quant(_nv_tensor_example(), "nv_tensor")
    assert r["outer"].tolist() == [2.0 ** -10]
    # block 1: RN(2.625 / 6) = 0.4375, / 2^-10 = 448 -> E4M3 0x7E; s_eff = 0.4375
    # block 2: RN(0.1875 / 6) = 0.03125 -> 32 -> 0x60; s_eff = 0.03125
    # block 3: RN(1.34375 / 6) / 2^-10 = 229.33 -> nearest E4M3 224 -> 0x76;
    #          s_eff = 224 * 2^-10 = 0.21875
    assert r["scales"].tolist() == [[0x7E, 0x60, 0x76]]
    c = unpack(r["codes"])[0]
    # a = 6, 1, 1.5, 0.25 (tie -> 0), 3.5 (tie -> 4), 5 (tie -> 4)
    assert c[0:6].tolist() == [0x7, 0x2, 0xB, 0x0, 0x6, 0x6]
    # a = 6, 1.5, 0.25 (tie -> 0, negative -> code 8)
    assert c[16:19].tolist() == [0x7, 0x3, 0x8]
    # a = 1.34375 / 0.21875 = 6.142857 -> 6 (clipped); 0.5 / 0.21875 = 2.2857 -> 2
    assert c[32:34].tolist() == [0x7, 0x4]
    y = f32(r["y"])[0]
    assert y[0:6].tolist() == [2.625, 0.4375, -0.65625, 0.0, 1.75, 1.75]
    assert y[16:19].tolist() == [0.1875, 0.046875, -0.0]
    assert np.signbit(y[18])
    assert y[32:34].tolist() == [1.3125, 0.4375]
    clip = r["clip"][0]
    assert np.flatnonzero(clip).tolist() == [32]


def test_nv_tensor_ste_masks_only_clipped():
    x = _nv_tensor_example()
    r = oracle.fake_quant(x, "nv_tensor")
    dy = bf([np.arange(1, 49, dtype=np.float32)])
    dx = oracle.ste_backward(x, r["scales"], r["outer"], dy, "nv_tensor")
    want = dy.copy()
    want[0, 32] = 0          # the clipped element gets +0
    assert dx.tolist() == want.tolist()


def test_nv_128_single_outer_block_equals_per_tensor():
    rng = np.random.default_rng(11)
    x = bf(rng.standard_normal((5, 128)).astype(np.float32))
    for i in range(5):
        row = x[i:i + 1]
        t = oracle.fake_quant(row, "nv_tensor")
        d = oracle.fake_quant(row, "nv_128")
        assert t["codes"].tolist() == d["codes"].tolist()
        assert t["scales"].tolist() == d["scales"].tolist()
        assert t["y"].tolist() == d["y"].tolist()
        assert t["outer"][0] == d["outer"][0, 0]


def test_all_zero_tensor():
    x = np.zeros((2, 128), np.uint16)
    x[1, 5] = 0x8000    # -0.0
    for fmt in ("mx", "nv_tensor", "nv_128"):
        r = oracle.fake_quant(x, fmt)
        assert np.all(unpack(r["codes"])[0] == 0)
        assert unpack(r["codes"])[1, 5] == 8
        assert np.all((r["y"] & 0x7FFF) == 0)
        assert r["y"][1, 5] == 0x8000
        assert not r["clip"].any()
    assert oracle.fake_quant(x, "mx")["scales"].max() == 0       # 2^-127
    assert oracle.fake_quant(x, "nv_tensor")["outer"][0] == 0.0


def test_sr_worked_examples_at_tensor_level():
    # MX block with amax 7 (scale 1): x = 0.30078125 rounds to 0.5 with
    # probability 39424 / 65536; x = 5.5 to 6 with probability 3/4; x = 7 -> 6.
    n = 4096
    vals = np.zeros((n, 32), np.float32)
    vals[:, 0] = 7.0
    vals[:, 1] = 0.30078125
    vals[:, 2] = 5.5
    r = oracle.fake_quant(bf(vals), "mx", "sr", seed=99)
    y = f32(r["y"])
    assert np.all(y[:, 0] == 6.0)
    p1 = (y[:, 1] == 0.5).mean()
    p2 = (y[:, 2] == 6.0).mean()
    assert set(np.unique(y[:, 1]).tolist()) <= {0.0, 0.5}
    assert set(np.unique(y[:, 2]).tolist()) <= {4.0, 6.0}
    se = 0.5 / np.sqrt(n)
    assert abs(p1 - 39424 / 65536) < 5 * se
    assert abs(p2 - 0.75) < 5 * se


def test_keep_mask_worked_block():
    # the worked MX block: only element 7 (-7, a = 7 > 6) is clipped, so bit 7
    # of byte 0 is clear and every other bit of the 32 elements is set
    x = [1, -0.30078125, 5.5, 0.25, -2.5, 0.75, 3.5, -7, 1.25, -1.75, 5] + [0] * 21
    r = oracle.fake_quant(bf([x]), "mx")
    assert oracle.keep_mask(r["clip"]).tolist() == [[0x7F, 0xFF, 0xFF, 0xFF]]
    dy = bf([np.arange(1, 33, dtype=np.float32)])
    dx = oracle.ste_backward_mask(oracle.keep_mask(r["clip"]), dy)
    want = dy.copy()
    want[0, 7] = 0
    assert dx.tolist() == want.tolist()


def test_keep_mask_nv_tensor_worked_block():
    # the clipped element of the NVFP4 example is element 32 (a = 6.142857):
    # byte 4, bit 0
    x = _nv_tensor_example()
    r = oracle.fake_quant(x, "nv_tensor")
    k = oracle.keep_mask(r["clip"])[0].tolist()
    assert k == [0xFF] * 4 + [0xFE, 0xFF]


def test_keep_mask_ste_equals_recomputed_ste():
    # The mask is taken from the forward's own quotients; ste_backward
    # recomputes a from the stored scale codes.  Both must pass the same
    # gradients, on every format and axis, on data that clips.
    from workloads import activation_with_outlier_channels, grad_output
    x = activation_with_outlier_channels((256, 384), 1.0, 6, 100.0, seed=5)
    dy = grad_output(256, 384, seed=6)
    for fmt in ("mx", "nv_tensor", "nv_128"):
        for axis in ("row", "col"):
            for rnd in ("rne", "sr"):
                r = oracle.fake_quant(x, fmt, rnd, axis, seed=9)
                assert r["clip"].any()
                want = oracle.ste_backward(x, r["scales"], r["outer"], dy, fmt, axis)
                got = oracle.ste_backward_mask(oracle.keep_mask(r["clip"]), dy)
                assert np.array_equal(got, want), (fmt, axis, rnd)
