"""Pins of the oracle's random Hadamard transform (TetraJet-v2 sec. 2.C).

- The n = 128 normalization constant is the FP32 value nearest to
  1/sqrt(128) (checked against 60-digit decimal arithmetic).
- Basis vectors: the transform of e_j is s_j / sqrt(n) times column j of the
  Sylvester Hadamard matrix (scipy.linalg.hadamard), exactly, so the
  butterfly order, the sign flips and the scaling are each pinned.
- Small integers: the butterflies add integers exactly in FP32, so the result
  equals one FP32 rounding of c_n times the integer product with scipy's
  Hadamard matrix, then BF16 round-to-nearest-even.
- The transform is orthogonal: applying S * H^T / sqrt(n) in float64 to the
  output recovers the input up to the BF16 rounding of the output.
"""
import decimal

import numpy as np
import pytest
import scipy.linalg

import oracle


def _bf16_bits(v):
    """BF16 round-to-nearest-even of float32 values (finite)."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _signs(seed, n_pos):
    return np.array([-1.0 if oracle.rht_sign_bit(seed, j) else 1.0 for j in range(n_pos)])


def test_scale_128_is_nearest_fp32():
    decimal.getcontext().prec = 60
    target = decimal.Decimal(1) / decimal.Decimal(128).sqrt()
    bits = oracle.RHT_SCALE_BITS[128]
    cands = np.array([bits - 1, bits, bits + 1], dtype=np.uint32).view(np.float32)
    dist = [abs(decimal.Decimal(float(c)) - target) for c in cands]
    assert dist[1] < dist[0] and dist[1] < dist[2]
    assert oracle.rht_scale(16) == 0.25


@pytest.mark.parametrize("n", [16, 128])
def test_basis_vectors_give_signed_hadamard_columns(n):
    seed = 0x1234ABCD5678
    H = scipy.linalg.hadamard(n)
    s = _signs(seed, n)
    x = np.zeros((n, n), dtype=np.uint16)
    x[np.arange(n), np.arange(n)] = 0x3F80                       # row j = e_j (1.0)
    y = oracle.bf16_bits_to_f64(oracle.hadamard(x, n, "row", seed))
    c = oracle.rht_scale(n)
    want = _bf16_bits(np.float32(c) * (H.T * s[:, None]).astype(np.float32))
    assert np.array_equal(oracle.hadamard(x, n, "row", seed), want)
    if n == 16:
        assert np.array_equal(y, (H.T * s[:, None]) * 0.25)


@pytest.mark.parametrize("n", [16, 128])
def test_small_integers_match_the_matrix_product(n):
    rng = np.random.default_rng(5)
    R, C = 8, 2 * n
    xi = rng.integers(-3, 4, size=(R, C)).astype(np.float32)
    x = _bf16_bits(xi)
    seed = 99
    s = _signs(seed, C)
    H = scipy.linalg.hadamard(n).astype(np.int64)
    prod = np.concatenate([((xi[:, b:b + n] * s[b:b + n]).astype(np.int64)) @ H.T
                           for b in range(0, C, n)], axis=1)
    want = _bf16_bits(np.float32(oracle.rht_scale(n)) * prod.astype(np.float32))
    assert np.array_equal(oracle.hadamard(x, n, "row", seed), want)


@pytest.mark.parametrize("n", [16, 128])
def test_inverse_round_trip(n):
    rng = np.random.default_rng(7)
    xf = rng.standard_normal((16, 4 * n)).astype(np.float32)
    x = _bf16_bits(xf)
    seed = 2024
    y = oracle.bf16_bits_to_f64(oracle.hadamard(x, n, "row", seed))
    H = scipy.linalg.hadamard(n).astype(np.float64) / np.sqrt(n)
    s = _signs(seed, 4 * n)
    z = np.concatenate([(y[:, b:b + n] @ H) * s[b:b + n] for b in range(0, 4 * n, n)], axis=1)
    xd = oracle.bf16_bits_to_f64(x)
    assert np.linalg.norm(z - xd) / np.linalg.norm(xd) < 4e-3
    # column axis: the same transform of the transpose
    assert np.array_equal(oracle.hadamard(np.ascontiguousarray(x.T), n, "col", seed).T,
                          oracle.hadamard(x, n, "row", seed))
