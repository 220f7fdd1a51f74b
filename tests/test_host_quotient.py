"""Host-side proofs of the division steps the GPU quantizers use.

The kernels compute a = RN(|x| / s) per element as q = RN(|x| * rcp),
r = fma(-q, s, |x|), a = fma(r, rcp, q) with rcp = RN(1 / s) taken once per
block.  tests/host/quotient_check.c runs that sequence in IEEE binary32 on the
host for every BF16 significand of x against every FP32 significand of s
(2^30 pairs) and counts results that differ from the correctly rounded
quotient.  This checks the arithmetic design, not the GPU build; the GPU
parity tests compare the kernels themselves with the oracle.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _run_check(tmp_path, name):
    if shutil.which("gcc") is None:
        pytest.skip("gcc unavailable")
    flags = open("/proc/cpuinfo").read() if os.path.exists("/proc/cpuinfo") else ""
    if " fma " not in flags:
        pytest.skip("host CPU has no FMA instruction")
    exe = tmp_path / name
    subprocess.run(["gcc", "-O2", "-mfma", "-fopenmp", "-ffp-contract=off",
                    os.path.join(HERE, "host", name + ".c"), "-o", str(exe), "-lm"],
                   check=True)
    return subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)


def test_corrected_quotient_is_correctly_rounded(tmp_path):
    out = _run_check(tmp_path, "quotient_check")
    assert out.stdout.strip() == "0", out.stdout + out.stderr


def test_division_free_scale_chain(tmp_path):
    """RN(amax/6), RN(A/2688) by constant reciprocals and RN(p/s) by one
    corrected step equal IEEE division for every pair of BF16 maxima (where
    the E4M3 block scale can be non-zero)."""
    out = _run_check(tmp_path, "scale_chain_check")
    assert out.stdout.split() == ["0", "0", "0"], out.stdout + out.stderr
