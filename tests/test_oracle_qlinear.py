"""Pins of the oracle's QAT linear forward, Y = FQ(X, along K) @ FQ(W, along K).

The operands are built so that the expected fake-quantized tensors and the
product are known exactly without the oracle:

* every block along K holds values (g + d) * s, with g on the E2M1 grid,
  |d| <= 1/8 (so round-to-nearest moves the value back to g * s: every grid
  gap is at least 1/2), and one unperturbed element of magnitude 6 * s that
  fixes the block scale s (MXFP4: floor(log2(6 s)) - 2 = log2 s; NVFP4: the
  outer scale is a power of two 2^j because the largest block of the tensor,
  or of each 128-block, is 6 * 448 * 2^j, and the block scale is a power of
  two v, so every quotient in the scale chain is exact);
* the block scales change from block to block along both axes, so grouping W
  along N (its rows) instead of K (its columns), or X along M, mixes blocks of
  different scales and changes the result;
* X, W and the perturbations differ, so a linear that skips the quantization,
  transposes an operand or shares one operand's per-tensor scale with the
  other gives a different product.

The expected product is an exact integer matrix product of the scaled grid
values (numpy int64, no floating point), compared with the oracle's float64
product for equality: every term is a short dyadic number, so the float64 sum
is exact in any order.
"""
import numpy as np
import pytest

import oracle
from workloads import f32_to_bf16_bits

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
DELTAS = np.array([0.0, 1 / 16, 1 / 8, -1 / 16, -1 / 8])
BLOCK = {"mx": 32, "nv_tensor": 16, "nv_128": 16}


def _block_values(rng, B, s, perturb):
    """One block: exact fake-quant values g * s and the input (g + d) * s."""
    g = rng.choice(GRID[:7], size=B)
    d = rng.choice(DELTAS, size=B) if perturb else np.zeros(B)
    d = np.where(g == 0, np.abs(d), d)          # stay on the positive side of 0
    sign = rng.choice([-1.0, 1.0], size=B)
    p = rng.integers(B)
    g[p], d[p] = 6.0, 0.0                        # the block maximum, unperturbed
    return sign * g * s, sign * (g + d) * s


def _operand(Q, L, fmt, rng, j_tensor):
    """[Q, L] values blocked along L (the quantized orientation): returns
    (input, expected fake quantization) as float64 arrays."""
    B = BLOCK[fmt]
    x = np.zeros((Q, L))
    xhat = np.zeros((Q, L))
    nb = L // B
    if fmt == "nv_tensor":
        top = (rng.integers(Q), rng.integers(nb))            # the one 448 block
    for q in range(Q):
        if fmt == "nv_128":
            j_o = rng.integers(-6, -2, size=L // 128)         # outer scale 2^j_o per 128
            top_in = rng.integers(8, size=L // 128)           # its 448 inner block
        for b in range(nb):
            if fmt == "mx":
                s, perturb = 2.0 ** rng.integers(-5, 6), True
            elif fmt == "nv_tensor":
                big = (q, b) == top
                v = 448.0 if big else 2.0 ** rng.integers(-4, 5)
                s, perturb = v * 2.0 ** j_tensor, not big
            else:
                o = b // 8
                big = b % 8 == top_in[o]
                v = 448.0 if big else 2.0 ** rng.integers(-4, 5)
                s, perturb = v * 2.0 ** j_o[o], not big
            xhat[q, b * B:(b + 1) * B], x[q, b * B:(b + 1) * B] = _block_values(rng, B, s, perturb)
    bits = f32_to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), x)          # exactly representable
    return bits, x, xhat


def _to_int(a, lsb_exp):
    """a * 2^-lsb_exp as exact int64 (asserted to be integers below 2^23)."""
    v = a * 2.0 ** -lsb_exp
    assert np.array_equal(v, np.round(v)) and np.abs(v).max() < 2 ** 23
    return v.astype(np.int64)


@pytest.mark.parametrize("fmt", ["nv_tensor", "mx", "nv_128"])
def test_qlinear_exact_operands(fmt):
    M, K, N = 128, 256, 384
    rng = np.random.default_rng({"mx": 1, "nv_tensor": 2, "nv_128": 3}[fmt])
    xb, xv, xhat = _operand(M, K, fmt, rng, j_tensor=-3)           # X blocked along K
    wtb, wtv, whatt = _operand(N, K, fmt, rng, j_tensor=-9)        # W^T blocked along K
    wb = np.ascontiguousarray(wtb.T)
    what = whatt.T
    assert not np.array_equal(xv, xhat) and not np.array_equal(wtv, whatt)

    r = oracle.qlinear(xb, wb, fmt, fmt)
    got_x, got_w = oracle.bf16_bits_to_f64(r["xhat"]), oracle.bf16_bits_to_f64(r["what"])
    assert got_x.shape == (M, K) and got_w.shape == (K, N) and r["y"].shape == (M, N)
    assert np.array_equal(got_x, xhat)
    assert np.array_equal(got_w, what)

    # exact product: every value is a multiple of 2^-14 below 2^9, so the
    # int64 sums (K = 256 terms below 2^46) are exact and below 2^53
    yint = _to_int(xhat, -14) @ _to_int(what, -14)
    assert np.abs(yint).max() < 2 ** 53
    assert np.array_equal(r["y"], yint.astype(np.float64) * 2.0 ** -28)

    # the construction discriminates: the wrong grouping axis, no quantization
    # or a product of the unquantized operands all give other values
    assert not np.array_equal(
        oracle.bf16_bits_to_f64(oracle.fake_quant(wb, fmt, "rne", "row")["y"]), what)
    assert not np.array_equal(
        oracle.bf16_bits_to_f64(oracle.fake_quant(xb, fmt, "rne", "col")["y"]), xhat)
    assert not np.array_equal(xv @ wtv.T, r["y"])


def test_qlinear_worked_nvfp4():
    """One row of X and one column of W, K = 16, NVFP4 per tensor, by hand.

    X = [6, 1.5625, 3, -0.5625, 0 x 12] * 448 * 2^-10: A = 2.625, so
    s_t = RN(2.625 / 2688) = 2^-10; the block maximum gives
    RN(RN(2.625 / 6) / 2^-10) = 448 (E4M3 0x7E) and s_eff = 0.4375; the
    quotients 6, 1.5625, 3, 0.5625 round to 6, 1.5, 3, 0.5, so
    X_hat = [2.625, 0.65625, 1.3125, -0.21875, 0 ...].
    W = [4, -6, 1, 0.9375, 0 x 12]^T * 448 * 2^-8: A = 10.5, s_t = 2^-8,
    block scale 448, s_eff = 1.75; 0.9375 rounds to 1, so
    W_hat = [7, -10.5, 1.75, 1.75, 0 ...]^T.
    Y = 2.625 * 7 - 0.65625 * 10.5 + 1.3125 * 1.75 - 0.21875 * 1.75
      = 18.375 - 6.890625 + 2.296875 - 0.3828125 = 13.3984375.
    """
    xr = np.zeros((1, 16))
    xr[0, :4] = np.array([6, 1.5625, 3, -0.5625]) * 448 * 2.0 ** -10
    wc = np.zeros((16, 1))
    wc[:4, 0] = np.array([4, -6, 1, 0.9375]) * 448 * 2.0 ** -8
    xb = f32_to_bf16_bits(xr.astype(np.float32))
    wb = f32_to_bf16_bits(wc.astype(np.float32))
    assert np.array_equal(oracle.bf16_bits_to_f64(xb), xr)
    assert np.array_equal(oracle.bf16_bits_to_f64(wb), wc)
    r = oracle.qlinear(xb, wb, "nv_tensor", "nv_tensor")
    assert oracle.bf16_bits_to_f64(r["xhat"])[0, :4].tolist() == [2.625, 0.65625, 1.3125, -0.21875]
    assert oracle.bf16_bits_to_f64(r["what"])[:4, 0].tolist() == [7.0, -10.5, 1.75, 1.75]
    assert r["y"].tolist() == [[13.3984375]]
