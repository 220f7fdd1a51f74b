"""What the random Hadamard transform is for (TetraJet-v2 sec. 2.C): with
outlier channels along a backward product's contraction axis, rotating the
operands before FP4 quantization lowers the error of the product.  Measured
with the oracle on MXFP4 gradient operands, whose power-of-two block scales
leave the most room; the rotation cancels in the exact product, so the error
is taken against the unrotated float64 product."""
import numpy as np

import oracle
import workloads as wl


def _mean_dx_error(x, w, dy, fmt, rht, seeds):
    errs = []
    for t in seeds:
        r = oracle.qlinear_bwd(x, w, dy, "nv_tensor", "nv_tensor", fmt, "sr", 100 + 4 * t,
                               rht_block=rht, rht_seed=5 + t, nthreads=4)
        g = oracle.bf16_bits_to_f64(dy)
        exact = r["keep_x"] * (g @ oracle.bf16_bits_to_f64(r["what"]).T)
        errs.append(np.linalg.norm(r["dx"] - exact) / np.linalg.norm(exact))
    return float(np.mean(errs))


def test_rht_lowers_mxfp4_backward_error_with_outlier_channels():
    M, K, N = 128, 64, 512
    x = wl.normal_bf16((M, K), 1.0, 6)
    w = wl.normal_bf16((K, N), 0.02, 7)
    dy = wl.activation_with_outlier_channels((M, N), 1e-3, 4, 100.0, seed=8)
    plain = _mean_dx_error(x, w, dy, "mx", 0, range(6))
    rotated = _mean_dx_error(x, w, dy, "mx", 128, range(6))
    assert rotated < 0.92 * plain, (rotated, plain)


def test_rht_is_neutral_without_outliers():
    M, K, N = 128, 64, 512
    x = wl.normal_bf16((M, K), 1.0, 6)
    w = wl.normal_bf16((K, N), 0.02, 7)
    dy = wl.normal_bf16((M, N), 1e-3, 8)
    plain = _mean_dx_error(x, w, dy, "mx", 0, range(4))
    rotated = _mean_dx_error(x, w, dy, "mx", 128, range(4))
    assert abs(rotated - plain) < 0.05 * plain, (rotated, plain)
