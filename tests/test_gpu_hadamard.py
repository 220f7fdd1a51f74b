"""GPU parity of the random Hadamard transform (fq_hadamard) and of the QAT
linear backward with rotated operands: the transform bit-exact against the
oracle on both axes and both block sizes; the backward within 1e-2 relative
Frobenius error of the oracle's composition."""
import numpy as np
import pytest
import torch

import fp4_block_quantization_fq_amd as fq
import oracle
import workloads as wl
from gpu_util import make_desc, to_bits, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [16, 128])
@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("shape", [(256, 256), (384, 1024), (640, 136)])
def test_hadamard_bit_exact(n, axis, shape):
    R, C = shape
    q = C if axis == "row" else R
    if q % n:
        pytest.skip("axis not a multiple of the block")
    x = wl.activation_with_outlier_channels((R, C), 1.0, 4, 50.0, seed=21)
    seed = 0xC0FFEE + n
    print(f"hadamard {axis} n={n} {R}x{C}", flush=True)
    y = fq.fq_hadamard(to_dev(x), n, fq.FQ_AXIS_COL if axis == "col" else fq.FQ_AXIS_ROW, seed)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(y), oracle.hadamard(x, n, axis, seed))


def test_hadamard_full_size():
    x = wl.grad_output(8192, 5760, seed=8)
    for axis, ax in (("row", fq.FQ_AXIS_ROW), ("col", fq.FQ_AXIS_COL)):
        y = fq.fq_hadamard(to_dev(x), 128, ax, 77)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(y), oracle.hadamard(x, 128, axis, 77)), axis


@pytest.mark.parametrize("rht", [16, 128])
@pytest.mark.parametrize("M,K,N", [(128, 64, 256), (256, 96, 128)])
def test_qlinear_bwd_with_rht(rht, M, K, N):
    x = wl.normal_bf16((M, K), 1.0, 6)
    w = wl.normal_bf16((K, N), 0.02, 7)
    dy = wl.activation_with_outlier_channels((M, N), 1e-3, 3, 100.0, seed=8)
    ref = oracle.qlinear_bwd(x, w, dy, "nv_tensor", "nv_tensor", "nv_128", "sr", 1234,
                             rht_block=rht, rht_seed=55)
    dx, dw = fq.fq_qlinear_bwd(make_desc("nv_tensor"), make_desc("nv_tensor", "rne", "col"),
                               make_desc("nv_128", "sr", "row", 1234), to_dev(x), to_dev(w),
                               to_dev(dy), rht_block=rht, rht_seed=55)
    torch.cuda.synchronize()
    for name, got, keep in (("dx", dx, ref["keep_x"]), ("dw", dw, ref["keep_w"])):
        g = oracle.bf16_bits_to_f64(to_bits(got))
        assert np.all(g[keep == 0] == 0), name
        err = np.linalg.norm(g - ref[name]) / np.linalg.norm(ref[name])
        assert err < 4e-3, (name, err)
