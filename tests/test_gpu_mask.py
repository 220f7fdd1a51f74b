"""GPU parity of the bit-packed STE keep mask (fq_fake_quant_mask) and the
mask-driven STE (fq_ste_backward_mask): keep bits, codes, scales, outer
scales and y bit-exact against the oracle on every format, axis and
rounding, including a ragged last column tile and the full 16384x4096
workload; dx bit-exact against the oracle's mask STE, in and out of place."""
import numpy as np
import pytest
import torch

import fp4_block_quantization_fq_amd as fq
import oracle
import workloads as wl
from gpu_util import assert_same, make_desc, to_bits, to_dev, to_np

pytestmark = pytest.mark.gpu


def gpu_fake_quant_mask(x_bits, fmt, rnd, axis, seed):
    d = make_desc(fmt, rnd, axis, seed)
    x = to_dev(x_bits)
    R, C = x.shape
    out = fq.alloc_outputs(d, R, C, x.device)
    y, keep = fq.fq_fake_quant_mask(d, x, out=out)
    torch.cuda.synchronize()
    return {"y": to_bits(y), "codes": to_np(out.codes), "scales": to_np(out.scales),
            "outer": None if out.outer is None else to_np(out.outer), "keep": to_np(keep)}


def fits(fmt, axis, R, C):
    q = C if axis == "row" else R
    B = 32 if fmt == "mx" else 16
    return q % B == 0 and (fmt != "nv_128" or q % 128 == 0) and C % 8 == 0


@pytest.mark.parametrize("shape", [(256, 384), (384, 1024), (256, 4104)])
@pytest.mark.parametrize("rnd", ["rne", "sr"])
@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("fmt", ["mx", "nv_tensor", "nv_128"])
def test_fake_quant_mask_matches_oracle(fmt, axis, rnd, shape):
    R, C = shape
    if not fits(fmt, axis, R, C):
        pytest.skip("shape does not block for this format and axis")
    x = wl.activation_with_outlier_channels(shape, 1.0, 5, 100.0, seed=R + C)
    print(f"mask {fmt}/{axis}/{rnd} {R}x{C}", flush=True)
    ref = oracle.fake_quant(x, fmt, rnd, axis, seed=77)
    ref["keep"] = oracle.keep_mask(ref["clip"])
    assert (ref["keep"] != 0xFF).any()          # the data does clip somewhere
    got = gpu_fake_quant_mask(x, fmt, rnd, axis, seed=77)
    assert_same(got, ref, keys=("keep", "codes", "scales", "outer", "y"),
                tag=f"{fmt}/{axis}/{rnd}/{shape}")


@pytest.mark.parametrize("axis", ["row", "col"])
def test_fake_quant_mask_full_size(axis):
    x = wl.nv_activation(16384, 4096, seed=3)
    print(f"mask full size {axis}", flush=True)
    ref = oracle.fake_quant(x, "nv_128", "sr", axis, seed=1234)
    ref["keep"] = oracle.keep_mask(ref["clip"])
    got = gpu_fake_quant_mask(x, "nv_128", "sr", axis, seed=1234)
    assert_same(got, ref, keys=("keep", "codes", "scales", "outer", "y"), tag=f"full/{axis}")


@pytest.mark.parametrize("shape", [(64, 64), (129, 136), (16384, 4096)])
def test_ste_backward_mask_matches_oracle(shape):
    R, C = shape
    rng = np.random.default_rng(R * 7 + C)
    keep = rng.integers(0, 256, size=(R, C // 8), dtype=np.uint8)
    dy = wl.grad_output(R, C, seed=11)
    want = oracle.ste_backward_mask(keep, dy)
    tk, tdy = torch.from_numpy(keep).to("cuda:0"), to_dev(dy)
    dx = fq.fq_ste_backward_mask(tk, tdy)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(dx), want)
    fq.fq_ste_backward_mask(tk, tdy, dx=tdy)         # in place
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(tdy), want)


def test_mask_ste_equals_recomputing_ste():
    # the two STE paths on the GPU give the same dx
    x = wl.nv_activation(2048, 4096, seed=3)
    dy = wl.grad_output(2048, 4096, seed=4)
    d = make_desc("nv_128")
    tx, tdy = to_dev(x), to_dev(dy)
    out = fq.alloc_outputs(d, 2048, 4096, tx.device)
    _, keep = fq.fq_fake_quant_mask(d, tx, out=out)
    a = fq.fq_ste_backward(d, tx, out, tdy)
    b = fq.fq_ste_backward_mask(keep, tdy)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(a), to_bits(b))


def test_binding_checks_buffers():
    DEV = "cuda:0"
    # a buffer too small, a non-contiguous operand or the wrong element size
    # is refused before any launch
    x = torch.zeros((64, 256), dtype=torch.bfloat16, device=DEV)
    d = fq.fq_desc_nvfp4(outer=fq.FQ_OUTER_BLOCK128)
    with pytest.raises(ValueError, match="bytes"):
        fq.fq_fake_quant(d, x, y=torch.empty((32, 256), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError, match="contiguous"):
        fq.fq_fake_quant(d, torch.zeros((256, 64), dtype=torch.bfloat16, device=DEV).t())
    with pytest.raises(ValueError, match="element"):
        fq.fq_fake_quant(d, x.float())
    out = fq.alloc_outputs(d, 64, 256, DEV)
    out.codes = out.codes[:32]
    with pytest.raises(ValueError, match="codes"):
        fq.fq_fake_quant(d, x, out=out)
