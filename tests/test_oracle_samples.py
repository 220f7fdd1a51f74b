"""The oracle on samples cut from a larger tensor (index_base): a run of
whole rows, or one whole column, quantized on its own with the flat index of
its first element as the stochastic-rounding base gives exactly the rows or
the column of the whole tensor's quantization; and a base beyond 2^32 adds
to the element index as a 64-bit integer, element by element against the
definition (fixed draws r16(seed, index) and the E2M1 rounding rule)."""
import numpy as np
import pytest

import oracle
from workloads import normal_bf16

KEYS = ("codes", "scales", "outer", "y", "clip")


def _eq(a, b):
    return (a is None and b is None) or np.array_equal(a, b)


@pytest.mark.parametrize("fmt", ["mx", "nv_128"])
@pytest.mark.parametrize("rounding", ["rne", "sr"])
def test_row_samples_match_the_whole_tensor(fmt, rounding):
    R, C = 64, 256
    x = normal_bf16((R, C), 1.0, 41)
    full = oracle.fake_quant(x, fmt, rounding, "row", seed=77)
    for r0, n in ((0, 1), (5, 3), (63, 1)):
        s = oracle.fake_quant(x[r0:r0 + n], fmt, rounding, "row", seed=77, index_base=r0 * C)
        for k in ("codes", "scales", "y", "clip"):
            assert np.array_equal(s[k], full[k][r0:r0 + n]), (k, r0)
        if fmt == "nv_128":
            assert np.array_equal(s["outer"], full["outer"][r0:r0 + n])


@pytest.mark.parametrize("fmt", ["mx", "nv_128"])
def test_column_samples_match_the_whole_tensor(fmt):
    R, C = 256, 48
    x = normal_bf16((R, C), 1.0, 42)
    full = oracle.fake_quant(x, fmt, "sr", "col", seed=78)
    for c in (0, 17, 47):
        s = oracle.fake_quant(np.ascontiguousarray(x[:, c:c + 1]), fmt, "sr", "col", seed=78,
                              index_base=c * R)
        assert np.array_equal(s["codes"][0], full["codes"][c])
        assert np.array_equal(s["scales"][0], full["scales"][c])
        assert np.array_equal(s["y"][:, 0], full["y"][:, c])
        if fmt == "nv_128":
            assert np.array_equal(s["outer"][0], full["outer"][c])


def test_a_wrong_base_is_seen():
    """The sample check is not vacuous: off by one element, the draws differ."""
    R, C = 8, 256
    x = normal_bf16((R, C), 1.0, 43)
    full = oracle.fake_quant(x, "nv_128", "sr", "row", seed=79)
    s = oracle.fake_quant(x[3:4], "nv_128", "sr", "row", seed=79, index_base=3 * C + 1)
    assert not np.array_equal(s["codes"], full["codes"][3:4])


def test_base_beyond_2_32_against_the_definition():
    """One MXFP4 block (power-of-two scale, so a = |x| / s is exact) at flat
    index 2^33 + 2^32 + 32: every code is the stochastic rounding rule applied
    with the draw r16(seed, base + c)."""
    base = (1 << 33) + (1 << 32) + 32
    seed = 1234
    x = normal_bf16((1, 32), 1.0, 44)
    q = oracle.fake_quant(x, "mx", "sr", "row", seed=seed, index_base=base)
    f = np.array([oracle.bf16_to_f32(int(v)) for v in x[0]])
    amax = float(np.max(np.abs(f)))
    s_eff = oracle.e8m0_decode(oracle.mx_scale_code(amax))
    codes = np.empty(32, np.uint8)
    codes[0::2] = q["codes"][0] & 15
    codes[1::2] = q["codes"][0] >> 4
    for c in range(32):
        a = abs(f[c]) / s_eff
        m = oracle.e2m1_sr(a, oracle.r16(seed, base + c))
        assert codes[c] == ((8 if np.signbit(f[c]) else 0) | m), c
    # and the draws there are not those of the index modulo 2^32
    assert any(oracle.r16(seed, base + c) != oracle.r16(seed, (base + c) % (1 << 32))
               for c in range(32))
