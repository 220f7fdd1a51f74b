"""Helpers shared by the GPU tests: BF16 bit-pattern transfer and descriptor
construction.  No quantization arithmetic lives here."""
import numpy as np
import torch

import fp4_block_quantization_fq_amd as fq

DEV = "cuda:0"


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 BF16 bit patterns (host) -> torch.bfloat16 on the GPU."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(DEV)


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def make_desc(fmt: str, rounding: str = "rne", axis: str = "row", seed: int = 0):
    r = fq.FQ_ROUND_SR if rounding == "sr" else fq.FQ_ROUND_RNE
    a = fq.FQ_AXIS_COL if axis == "col" else fq.FQ_AXIS_ROW
    if fmt == "mx":
        return fq.fq_desc_mxfp4(rounding=r, axis=a, seed=seed)
    outer = fq.FQ_OUTER_TENSOR if fmt == "nv_tensor" else fq.FQ_OUTER_BLOCK128
    return fq.fq_desc_nvfp4(rounding=r, axis=a, seed=seed, outer=outer)


def gpu_fake_quant(x_bits, fmt, rounding="rne", axis="row", seed=0, with_outputs=True):
    """Run fq_fake_quant on the GPU; returns host numpy arrays."""
    d = make_desc(fmt, rounding, axis, seed)
    x = to_dev(x_bits)
    R, C = x.shape
    out = fq.alloc_outputs(d, R, C, x.device) if with_outputs else None
    y = fq.fq_fake_quant(d, x, out=out)
    torch.cuda.synchronize()
    res = {"y": to_bits(y)}
    if with_outputs:
        res["codes"] = to_np(out.codes)
        res["scales"] = to_np(out.scales)
        res["outer"] = None if out.outer is None else to_np(out.outer)
    return res


def assert_same(gpu: dict, ref: dict, keys=("codes", "scales", "outer", "y"), tag=""):
    for k in keys:
        g, r = gpu.get(k), ref.get(k)
        if r is None and g is None:
            continue
        assert g is not None and r is not None, (tag, k)
        g = np.asarray(g)
        r = np.asarray(r)
        assert g.shape == r.shape, (tag, k, g.shape, r.shape)
        if g.dtype == np.float32:
            g, r = g.view(np.uint32), r.view(np.uint32)
        bad = np.flatnonzero(g.reshape(-1) != r.reshape(-1))
        assert bad.size == 0, (f"{tag}: {k}: {bad.size} of {g.size} differ; first at flat "
                               f"{bad[:5].tolist()}: gpu {g.reshape(-1)[bad[:5]].tolist()} "
                               f"oracle {r.reshape(-1)[bad[:5]].tolist()}")


def assert_product_bound(got: np.ndarray, ref: np.ndarray, absprod: np.ndarray, kdim: int,
                         keep: np.ndarray | None = None, tag: str = ""):
    """Element-wise check of a BF16 matrix product against the float64 product
    `ref` of the same BF16 operands.  The products of BF16 values are exact in
    FP32, so the device result differs from `ref` only by the FP32
    accumulation (at most about kdim * 2^-24 * (|A| @ |B|), any order) and the
    final BF16 rounding (2^-8 relative): |got - ref| <= 2^-8 |ref| +
    2 kdim 2^-24 (|A| @ |B|).  Where keep is 0 the result must be +0 or -0."""
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 * kdim * 2.0 ** -24 * absprod
    err = np.abs(got - ref)
    if keep is not None:
        assert np.all(got[keep == 0] == 0), (tag, "dropped entries must be 0")
        err = np.where(keep == 0, 0.0, err)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (f"{tag}: {len(bad)} of {got.size} elements outside the bound; "
                           f"first {bad[:3].tolist()}: got {got[tuple(bad[0])]} ref "
                           f"{ref[tuple(bad[0])]} bound {bound[tuple(bad[0])]}")
