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
@pytest.mark.parametrize("shape", [(256, 256), (384, 1024), (640, 136), (16, 8), (48, 72),
                                   (128, 8), (272, 200)])
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


@pytest.mark.parametrize("rnd", ["rne", "sr"])
@pytest.mark.parametrize("n", [16, 128])
@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("fmt", ["mx", "nv_128"])
@pytest.mark.parametrize("shape", [(256, 384), (384, 1024)])
def test_fake_quant_rht_matches_oracle(fmt, axis, n, rnd, shape):
    # the fused rotate-and-quantize pass equals the oracle's quantizer applied
    # to the oracle's rotation, bit for bit
    R, C = shape
    x = wl.activation_with_outlier_channels(shape, 1.0, 4, 50.0, seed=R + n)
    print(f"fq_rht {fmt}/{axis}/n={n}/{rnd} {R}x{C}", flush=True)
    hx = oracle.hadamard(x, n, axis, 0xBEEF)
    ref = oracle.fake_quant(hx, fmt, rnd, axis, seed=99)
    d = make_desc(fmt, rnd, axis, 99)
    tx = to_dev(x)
    out = fq.alloc_outputs(d, R, C, tx.device)
    y = fq.fq_fake_quant_rht(d, tx, n, 0xBEEF, out=out)
    torch.cuda.synchronize()
    got = {"y": to_bits(y), "codes": out.codes.cpu().numpy(), "scales": out.scales.cpu().numpy(),
           "outer": None if out.outer is None else out.outer.cpu().numpy()}
    for k in ("codes", "scales", "outer", "y"):
        if ref[k] is None:
            continue
        g, r = np.asarray(got[k]), np.asarray(ref[k])
        if g.dtype == np.float32:
            g, r = g.view(np.uint32), r.view(np.uint32)
        assert np.array_equal(g, r), (fmt, axis, n, rnd, k)


def test_fake_quant_rht_full_size():
    x = wl.grad_output(8192, 5760, seed=8)
    for axis in ("row", "col"):
        hx = oracle.hadamard(x, 128, axis, 5)
        ref = oracle.fake_quant(hx, "nv_128", "sr", axis, seed=1234)
        d = make_desc("nv_128", "sr", axis, 1234)
        y = fq.fq_fake_quant_rht(d, to_dev(x), 128, 5)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(y), ref["y"]), axis


def test_qlinear_bwd_mxfp4_with_rht():
    x = wl.normal_bf16((256, 256), 1.0, 6)
    w = wl.normal_bf16((256, 384), 0.02, 7)
    dy = wl.activation_with_outlier_channels((256, 384), 1e-3, 3, 100.0, seed=8)
    ref = oracle.qlinear_bwd(x, w, dy, "mx", "mx", "mx", "sr", 1234, rht_block=128, rht_seed=55)
    dx, dw = fq.fq_qlinear_bwd(make_desc("mx"), make_desc("mx", "rne", "col"),
                               make_desc("mx", "sr", "row", 1234), to_dev(x), to_dev(w),
                               to_dev(dy), rht_block=128, rht_seed=55)
    torch.cuda.synchronize()
    for name, got, keep in (("dx", dx, ref["keep_x"]), ("dw", dw, ref["keep_w"])):
        g = oracle.bf16_bits_to_f64(to_bits(got))
        assert np.all(g[keep == 0] == 0), name
        err = np.linalg.norm(g - ref[name]) / np.linalg.norm(ref[name])
        assert err < 4e-3, (name, err)
