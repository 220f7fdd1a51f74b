"""fq_fake_quant_noalloc (no allocation, library-owned per-GPU scratch)
against fq_fake_quant with a caller workspace: bit-identical outputs, on two
calls in a row, the second with a smaller input, for every format and both
axes (the per-tensor NVFP4 format is the one that uses the scratch)."""
import numpy as np
import pytest
import torch

import fp4_block_quantization_fq_amd as fq
import workloads as wl
from gpu_util import assert_same, make_desc, to_bits, to_dev, to_np

pytestmark = pytest.mark.gpu


def _run(fn, d, x):
    R, C = x.shape
    out = fq.alloc_outputs(d, R, C, x.device)
    y = torch.empty_like(x)
    fn(d, x, y, out)
    torch.cuda.synchronize()
    return {"y": to_bits(y), "codes": to_np(out.codes), "scales": to_np(out.scales),
            "outer": None if out.outer is None else to_np(out.outer)}


def _with_ws(d, x, y, out):
    fq.fq_fake_quant(d, x, y=y, out=out)


def _noalloc(d, x, y, out):
    fq.fq_fake_quant_noalloc(d, x, y, out)


@pytest.mark.parametrize("fmt", ["nv_tensor", "mx", "nv_128"])
@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("rnd", ["rne", "sr"])
def test_noalloc_matches_workspace_call(fmt, axis, rnd):
    d = make_desc(fmt, rnd, axis, seed=99)
    # a large call (its maximum pass uses every partial) then a smaller one
    # with a smaller maximum, so a stale partial from the first would show
    big = wl.weight_with_outlier_entries((4096, 4096), 0.02, 1e-3, 50.0, seed=11)
    small = wl.normal_bf16((384, 256), 0.5, seed=12)
    for x in (big, small):
        xd = to_dev(x)
        assert_same(_run(_noalloc, d, xd), _run(_with_ws, d, xd),
                    tag=f"noalloc {fmt}/{axis}/{rnd} {x.shape}")
