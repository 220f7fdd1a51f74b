"""Pins for the oracle's element and scale encodings.

Each test checks the oracle against something other than itself: a published
table (golden file), a library conversion (torch float8 / bfloat16 casts), an
independent formulation (nearest-value search, bit-field decode, frexp), or
exhaustive enumeration.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle


def _read_golden(path):
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- E2M1 ----

def test_e2m1_decode_matches_published_grid(golden_dir):
    rows = _read_golden(os.path.join(golden_dir, "e2m1_grid.txt"))
    assert len(rows) == 16
    for code_s, val_s in rows:
        code, val = int(code_s, 16), float(val_s)
        got = oracle.e2m1_decode(code)
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code


def test_e2m1_decode_matches_bit_fields():
    # sign | 2-bit exponent (bias 1) | 1-bit mantissa; exponent 0 is subnormal
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        mag = (m * 0.5) if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
        assert oracle.e2m1_decode(code) == (-mag if s else mag)


def _all_finite_nonneg_bf16():
    u = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)  # +0 .. max finite
    return u, (u.astype(np.uint32) << 16).view(np.float32)


def test_e2m1_rne_threshold_table_all_bf16():
    """Every non-negative finite BF16 magnitude at unit scale against the
    threshold table derived by hand from round-to-nearest-even on the grid
    {0, .5, 1, 1.5, 2, 3, 4, 6}: ties at .25, .75, 1.25, 1.75, 2.5, 3.5, 5
    go to the even code, everything above 5 saturates at 6."""
    _, vals = _all_finite_nonneg_bf16()
    for a in vals:
        a = float(a)
        if a <= 0.25: want = 0
        elif a < 0.75: want = 1
        elif a <= 1.25: want = 2
        elif a < 1.75: want = 3
        elif a <= 2.5: want = 4
        elif a < 3.5: want = 5
        elif a <= 5.0: want = 6
        else: want = 7
        assert oracle.e2m1_rne(a) == want, a


def test_e2m1_rne_against_argmin_with_even_ties():
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    rng = np.random.default_rng(0)
    vals = np.concatenate([rng.uniform(0, 8, 20000), np.arange(0, 8, 0.125),
                           (grid[1:] + grid[:-1]) / 2])
    for a in vals.astype(np.float32):
        d = np.abs(grid - float(a))
        cand = np.flatnonzero(d == d.min())
        want = cand[0] if len(cand) == 1 else [c for c in cand if c % 2 == 0][0]
        assert oracle.e2m1_rne(float(a)) == want, a


def test_e2m1_encode_decode_roundtrip():
    for m in range(8):
        assert oracle.e2m1_rne(oracle.e2m1_decode(m)) == m
        # a grid value never rounds up under stochastic rounding
        assert oracle.e2m1_sr(oracle.e2m1_decode(m), 0) == m


@pytest.mark.parametrize("a", [0.30078125, 5.5, 0.25, 1.0009765625, 3.9921875,
                               4.8125, 0.0009765625, 2.0])
def test_e2m1_sr_expectation_by_enumeration(a):
    """Enumerate all 65536 draws: the mean rounded value equals a exactly when
    the fraction times 2^16 is an integer, and is short by < gap * 2^-16
    otherwise (never above a)."""
    grid = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    total = 0.0
    for r in range(65536):
        total += grid[oracle.e2m1_sr(a, r)]
    mean = total / 65536
    k = max(i for i in range(7) if grid[i] <= a)
    gap = grid[k + 1] - grid[k]
    frac = (a - grid[k]) / gap
    if float(frac * 65536).is_integer():
        assert mean == a
    else:
        assert 0 <= a - mean < gap * 2.0 ** -16


def test_e2m1_sr_worked_thresholds():
    # a = 0.30078125 in [0, 0.5): frac 0.6015625, T = 39424
    assert oracle.e2m1_sr(0.30078125, 39423) == 1
    assert oracle.e2m1_sr(0.30078125, 39424) == 0
    # a = 5.5 in [4, 6): frac 0.75, T = 49152
    assert oracle.e2m1_sr(5.5, 49151) == 7
    assert oracle.e2m1_sr(5.5, 49152) == 6
    # a >= 6 clips deterministically
    for r in (0, 1, 65535):
        assert oracle.e2m1_sr(7.0, r) == 7
        assert oracle.e2m1_sr(6.0, r) == 7


# ---------------------------------------------------------------- E4M3 ----

def test_e4m3_decode_matches_torch():
    codes = torch.arange(0, 0x7F, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).float().tolist()
    for c, r in zip(range(0x7F), ref):
        assert oracle.e4m3_decode(c) == r, c
    assert math.isnan(oracle.e4m3_decode(0x7F))


def test_e4m3_encode_matches_torch_cast():
    """Round to nearest even with saturation at 448: torch's float8_e4m3fn
    cast of min(v, 448) (torch itself maps values past 464 to NaN)."""
    rng = np.random.default_rng(1)
    vals = [np.float32(2.0) ** rng.uniform(-14, 10, 30000).astype(np.float32)]
    exact = np.array([oracle.e4m3_decode(c) for c in range(0x7F)], np.float64)
    mids = (exact[1:] + exact[:-1]) / 2
    vals.append(exact.astype(np.float32))
    vals.append(mids.astype(np.float32))
    vals.append(np.nextafter(mids.astype(np.float32), np.float32(np.inf)))
    vals.append(np.nextafter(mids.astype(np.float32), np.float32(0)))
    vals.append(np.array([0, 2.0 ** -10, 2.0 ** -11, 2.0 ** -9, 448, 460, 464, 470,
                          479, 480, 1e6, 1e-30], np.float32))
    v = np.concatenate(vals).astype(np.float32)
    ref = torch.from_numpy(np.minimum(v, np.float32(448))).to(torch.float8_e4m3fn)
    ref = ref.view(torch.uint8).numpy()
    for x, r in zip(v, ref):
        assert oracle.e4m3_encode(float(x)) == r, float(x)


# ---------------------------------------------------------------- E8M0 ----

def test_e8m0_decode_matches_torch():
    codes = torch.arange(0, 255, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).float().tolist()
    for c, r in zip(range(255), ref):
        assert oracle.e8m0_decode(c) == r, c


def test_mx_scale_code_floor_log2_against_frexp():
    """code = clamp(floor(log2 amax) - 2, -127, 127) + 127 with floor(log2)
    from math.frexp, over every positive finite BF16 value (including
    subnormals) and zero."""
    u, vals = _all_finite_nonneg_bf16()
    for a in vals:
        a = float(a)
        if a == 0.0:
            want = 0
        else:
            _, e = math.frexp(a)
            want = min(max(e - 1 - 2, -127), 127) + 127
        assert oracle.mx_scale_code(a) == want, a


def test_mx_scale_brackets_block_max():
    """For an unclamped block, amax / scale lies in [4, 8)."""
    _, vals = _all_finite_nonneg_bf16()
    for a in vals[::7]:
        a = float(a)
        if a == 0.0:
            continue
        code = oracle.mx_scale_code(a)
        if code == 0:
            continue  # clamped at 2^-127
        r = a / oracle.e8m0_decode(code)
        assert 4.0 <= r < 8.0, a


# ---------------------------------------------------------------- BF16 ----

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 1 << 32, 200000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    # values between bf16 max and f32 max overflow in torch too (IEEE rule)
    ref = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy()
    ref = ref.view(np.uint16)
    for x, r in zip(v[:50000], ref[:50000]):
        assert oracle.f32_to_bf16(float(x)) == r
    # ties: low half exactly 0x8000
    hi = rng.integers(0, 0x7F7F, 5000, dtype=np.uint32)
    tie = ((hi << 16) | 0x8000).view(np.float32)
    ref = torch.from_numpy(tie.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for x, r in zip(tie, ref):
        assert oracle.f32_to_bf16(float(x)) == r


def test_bf16_widening_exact():
    for h in (0x0000, 0x8000, 0x0001, 0x3F80, 0xBF80, 0x7F7F, 0x4040):
        f = np.array([h], np.uint16).astype(np.uint32) << 16
        assert oracle.bf16_to_f32(h) == float(f.view(np.float32)[0])


# ------------------------------------------------------- NV outer scale ----

def test_nv_outer_scale_is_amax_over_6_times_448():
    # hand-derived exact cases: 2688 = 6 * 448 = 128 * 21
    assert oracle.nv_outer_scale(2.625) == 2.0 ** -10     # 21/8 / (128*21)
    assert oracle.nv_outer_scale(1.3125) == 2.0 ** -11    # 21/16
    assert oracle.nv_outer_scale(2688.0) == 1.0
    assert oracle.nv_outer_scale(5376.0) == 2.0
    assert oracle.nv_outer_scale(0.0) == 0.0
    # 1 / 2688 is not a binary32 value: the result is the nearer neighbour
    s = oracle.nv_outer_scale(1.0)
    lo, hi = np.float32(s), np.nextafter(np.float32(s), np.float32(1))
    assert abs(float(lo) - 1 / 2688) <= abs(float(hi) - 1 / 2688)
    assert abs(float(lo) - 1 / 2688) <= abs(float(np.nextafter(lo, np.float32(0))) - 1 / 2688)
