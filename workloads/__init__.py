"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no quantization arithmetic: it only draws random tensors
and rounds them to BF16 (the input dtype).  Both the CPU oracle and the GPU
library are fed the same BF16 bit patterns produced here.

Recipe: numpy PCG64 (`numpy.random.default_rng(seed)`), float32
standard-normal draws times sigma, then the structure of the workload
(outlier entries or outlier channels), then round-to-nearest-even to BF16.
Shapes follow LLM linear layers: 2880 and 5760 are the hidden and MLP widths
of the gpt-oss family; 4096-wide layers and 16384-token activations follow
the TetraJet-v2 style activation quantizer.
"""
from __future__ import annotations

import numpy as np


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bit patterns (uint16), round to nearest even.

    Inputs here are finite by construction; the rounding is the usual
    add-half-minus-lsb on the 32-bit word.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) >> 16
    return u.astype(np.uint16)


def normal_bf16(shape, sigma: float, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)
    return f32_to_bf16_bits(a)


def weight_with_outlier_entries(shape, sigma: float, frac: float, factor: float,
                                seed: int) -> np.ndarray:
    """N(0, sigma^2) with round(frac * numel) entries (chosen without
    replacement) multiplied by `factor`."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)
    n = a.size
    k = int(round(frac * n))
    idx = rng.choice(n, size=k, replace=False)
    flat = a.reshape(-1)
    flat[idx] *= np.float32(factor)
    return f32_to_bf16_bits(a)


def activation_with_outlier_channels(shape, sigma: float, n_channels: int,
                                     factor: float, seed: int) -> np.ndarray:
    """N(0, sigma^2) with `n_channels` columns (chosen without replacement)
    multiplied by `factor`."""
    return activation_and_outlier_channels(shape, sigma, n_channels, factor, seed)[0]


def activation_and_outlier_channels(shape, sigma: float, n_channels: int, factor: float,
                                    seed: int):
    """activation_with_outlier_channels and the indices of the scaled columns."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)
    cols = rng.choice(shape[1], size=n_channels, replace=False)
    a[:, cols] *= np.float32(factor)
    return f32_to_bf16_bits(a), np.sort(cols)


# --------------------------------------------------------------------------
# The workloads (seed, shape, distribution, structure)
# --------------------------------------------------------------------------

def mx_activation(rows=1024, cols=4096, seed=1):
    """MXFP4 RNE workload: N(0, 1)."""
    return normal_bf16((rows, cols), 1.0, seed)


def nv_weight(rows=2880, cols=2880, seed=2):
    """NVFP4 per-tensor workload: N(0, 0.02^2), 0.1 % of entries x50."""
    return weight_with_outlier_entries((rows, cols), 0.02, 1e-3, 50.0, seed)


def nv_activation(rows=16384, cols=4096, seed=3):
    """Double-block NVFP4 workload: N(0, 1) with 8 outlier channels x100."""
    return activation_with_outlier_channels((rows, cols), 1.0, 8, 100.0, seed)


def grad_output(rows=16384, cols=4096, seed=4):
    """Upstream gradient for the STE backward: N(0, (1e-3)^2)."""
    return normal_bf16((rows, cols), 1e-3, seed)


def backward_weight(rows=4096, cols=4096, seed=5):
    """Weight quantized along the transposed axis: N(0, 0.02^2)."""
    return normal_bf16((rows, cols), 0.02, seed)


def linear_inputs(M=8192, K=2880, N=5760, seed_x=6, seed_w=7):
    """QAT linear: X [M, K] ~ N(0, 1), W [K, N] ~ N(0, 0.02^2)."""
    return normal_bf16((M, K), 1.0, seed_x), normal_bf16((K, N), 0.02, seed_w)


def uniform_bits_bf16(shape, seed: int) -> np.ndarray:
    """Random finite BF16 bit patterns of every exponent (edge-case sweeps)."""
    rng = np.random.default_rng(seed)
    u = rng.integers(0, 1 << 16, size=shape, dtype=np.uint32).astype(np.uint16)
    finite = (u & 0x7F80) != 0x7F80
    return np.where(finite, u, u & 0x807F).astype(np.uint16)


def device_normal_bf16(rows: int, cols: int, sigma: float, seed: int, device,
                       block_elems: int = 1 << 28):
    """A [rows, cols] BF16 tensor on `device`, N(0, sigma^2) drawn by torch's
    seeded device generator in blocks of whole rows and rounded by torch's
    BF16 cast: for tensors too large to draw on the host (beyond 2^32
    elements).  Whoever uses it copies sampled rows or columns to the host
    for the oracle."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.empty((rows, cols), dtype=torch.bfloat16, device=device)
    step = max(1, block_elems // cols)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        blk = torch.randn((r1 - r0, cols), generator=g, device=device, dtype=torch.float32)
        x[r0:r1] = (blk * sigma).to(torch.bfloat16)
        del blk
    return x
