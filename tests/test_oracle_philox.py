"""Pins for the oracle's counter-based generator (Philox4x32-10) and the
mapping of its output words to per-element 16-bit draws."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle


def test_philox_known_answer_vectors(golden_dir):
    n = 0
    with open(os.path.join(golden_dir, "philox4x32_10_kat.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            w = [int(t, 16) for t in line.split()]
            assert oracle.philox4x32_10(w[0:4], w[4:6]) == w[6:10]
            n += 1
    assert n == 3


_TORCH_PROBE = r"""
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cstdint>
int main() {
  unsigned long long seed, offset;
  while (std::scanf("%llu %llu", &seed, &offset) == 2) {
    at::philox_engine e(seed, 0, offset);
    unsigned a = e(), b = e(), c = e(), d = e();
    std::printf("%u %u %u %u\n", a, b, c, d);
  }
  return 0;
}
"""


def test_philox_matches_torch_engine(tmp_path):
    """Cross-check against PyTorch's host Philox4x32-10 engine (public header
    source, compiled here): key = seed, counter = (offset, subsequence 0)."""
    import torch
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    if shutil.which("g++") is None or not os.path.exists(
            os.path.join(inc, "ATen", "core", "PhiloxRNGEngine.h")):
        pytest.skip("g++ or torch headers unavailable")
    src = tmp_path / "probe.cpp"
    exe = tmp_path / "probe"
    src.write_text(_TORCH_PROBE)
    r = subprocess.run(["g++", "-std=c++17", "-O1", f"-I{inc}", str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("torch Philox header did not compile: " + r.stderr[:200])
    rng = np.random.default_rng(7)
    cases = [(0, 0), (1234, 0), (1234, 1), (1235, 7), (2**64 - 1, 2**40 + 3)]
    cases += [(int(s), int(o)) for s, o in zip(rng.integers(0, 2**63, 40, dtype=np.uint64),
                                               rng.integers(0, 2**40, 40, dtype=np.uint64))]
    inp = "".join(f"{s} {o}\n" for s, o in cases)
    out = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True)
    for (s, o), line in zip(cases, out.stdout.strip().splitlines()):
        want = [int(t) for t in line.split()]
        got = oracle.philox4x32_10([o & 0xFFFFFFFF, o >> 32, 0, 0],
                                   [s & 0xFFFFFFFF, s >> 32])
        assert got == want, (s, o)


def test_r16_index_mapping():
    """Element n uses call n >> 3, word (n >> 1) & 3, low half for even n."""
    seed = 0x0123456789ABCDEF
    for n in [0, 1, 2, 7, 8, 13, 15, 4095, 4096, 2**33 + 5]:
        call = n >> 3
        o = oracle.philox4x32_10([call & 0xFFFFFFFF, call >> 32, 0, 0],
                                 [seed & 0xFFFFFFFF, seed >> 32])
        w = o[(n >> 1) & 3]
        want = (w >> 16) if (n & 1) else (w & 0xFFFF)
        assert oracle.r16(seed, n) == want, n
    # element 13: call 1, word 2, high half
    o = oracle.philox4x32_10([1, 0, 0, 0], [seed & 0xFFFFFFFF, seed >> 32])
    assert oracle.r16(seed, 13) == o[2] >> 16


def test_r16_statistics():
    """Bit balance and a chi-square test of the 16-bit draws (first 2^15
    indices, seed 1234) over 256 equal bins."""
    draws = np.array([oracle.r16(1234, n) for n in range(1 << 15)], np.uint32)
    bits = ((draws[:, None] >> np.arange(16)) & 1).mean(axis=0)
    assert np.all(np.abs(bits - 0.5) < 0.02)
    hist = np.bincount(draws >> 8, minlength=256)
    expected = len(draws) / 256
    chi2 = float(((hist - expected) ** 2 / expected).sum())
    # 255 degrees of freedom: mean 255, sd ~22.6; reject only far tails
    assert 160 < chi2 < 370, chi2
