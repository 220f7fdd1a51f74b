"""Pins of the oracle's QAT linear backward (a composition of pinned pieces).

1. Exact operands.  MXFP4 inputs whose every 32-element block, along both
   axes, holds values on the E2M1 grid with a +-6 in it: every quantization
   in the backward is then the identity (stochastic rounding of a grid value
   never moves it), so dX and dW must equal the plain float64 products
   dY @ W^T and X^T @ dY exactly.  A transposed operand or a product taken
   along the wrong axis fails this.
2. Unbiasedness (TetraJet-v2 sec. 2.A: stochastic rounding makes
   E[round(x)] = x in the backward).  Over many seeds the mean of dX tends to
   keep_X * (dY @ W_hat^T) and the mean of dW to keep_W * (X_hat^T @ dY),
   where X_hat, W_hat are the forward's operands; the distance to the same
   products taken with the unquantized X and W stays large, so a backward
   that used X instead of X_hat would fail.
"""
import numpy as np
import pytest

import oracle

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _grid_tensor(R, C, seed):
    """Values g * 2^0 with a 6 wherever (i + j) % 32 == 0 (so every 32-block
    along either axis has amax 6 and E8M0 scale 1)."""
    rng = np.random.default_rng(seed)
    v = rng.choice(GRID, size=(R, C)) * rng.choice([-1.0, 1.0], size=(R, C))
    i, j = np.indices((R, C))
    v[(i + j) % 32 == 0] = 6.0
    bits = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), v)     # exactly representable
    return bits, v


def test_exact_operands_give_plain_products():
    M, K, N = 64, 96, 64
    xb, xv = _grid_tensor(M, K, 1)
    wb, wv = _grid_tensor(K, N, 2)
    gb, gv = _grid_tensor(M, N, 3)
    r = oracle.qlinear_bwd(xb, wb, gb, fmt_x="mx", fmt_w="mx", fmt_g="mx",
                           rounding_g="sr", seed_g=77)
    assert np.array_equal(r["keep_x"], np.ones_like(xv))
    assert np.array_equal(r["keep_w"], np.ones_like(wv))
    assert np.array_equal(r["dx"], gv @ wv.T)
    assert np.array_equal(r["dw"], xv.T @ gv)


def _unclipped_bits(shape, seed):
    """Uniform values in [-1.25, 1.25] with a +1.25 wherever (i + j) % 16 == 0:
    every 16- and 32-element block along either axis has amax 1.25, so no
    element is clipped (MXFP4: a <= 1.25 / 2^-2 = 5; NVFP4 per-tensor: the
    block scale is 448 * s_t = 1.25 / 6 up to one rounding), and stochastic
    rounding is unbiased for every element."""
    rng = np.random.default_rng(seed)
    f = rng.uniform(-1.25, 1.25, size=shape).astype(np.float32)
    i, j = np.indices(shape)
    f[(i + j) % 16 == 0] = 1.25
    return (f.view(np.uint32) >> 16).astype(np.uint16)     # truncation keeps |v| <= 1.25


@pytest.mark.parametrize("fmt", ["mx", "nv_tensor"])
def test_stochastic_backward_is_unbiased(fmt):
    M, K, N = 64, 64, 64
    x = _unclipped_bits((M, K), 11)
    w = _unclipped_bits((K, N), 12)
    dy = _unclipped_bits((M, N), 13)
    T = 256
    acc_dx = np.zeros((M, K))
    acc_dw = np.zeros((K, N))
    one = None
    for t in range(T):
        r = oracle.qlinear_bwd(x, w, dy, fmt_x=fmt, fmt_w=fmt, fmt_g=fmt, rounding_g="sr",
                               seed_g=1000 + 4 * t, nthreads=1)
        acc_dx += r["dx"]
        acc_dw += r["dw"]
        one = one or r
    xh = oracle.bf16_bits_to_f64(one["xhat"])
    wh = oracle.bf16_bits_to_f64(one["what"])
    g = oracle.bf16_bits_to_f64(dy)
    want_dx = one["keep_x"] * (g @ wh.T)
    want_dw = one["keep_w"] * (xh.T @ g)
    rel = lambda a, b: np.linalg.norm(a - b) / np.linalg.norm(b)
    assert one["keep_x"].all() and one["keep_w"].all()
    single = rel(one["dx"], want_dx)
    assert rel(acc_dx / T, want_dx) < 0.15 * single       # noise shrinks like 1/sqrt(T)
    assert rel(acc_dx / T, want_dx) < 0.02
    assert rel(acc_dw / T, want_dw) < 0.02
    # the forward's quantization error is far above that noise floor
    wrong_dw = one["keep_w"] * (oracle.bf16_bits_to_f64(x).T @ g)
    assert rel(acc_dw / T, wrong_dw) > 0.05
