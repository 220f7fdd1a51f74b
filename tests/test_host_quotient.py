"""Host-side proof of the division step the GPU quantizers use.

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


def test_corrected_quotient_is_correctly_rounded(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc unavailable")
    flags = open("/proc/cpuinfo").read() if os.path.exists("/proc/cpuinfo") else ""
    if " fma " not in flags:
        pytest.skip("host CPU has no FMA instruction")
    exe = tmp_path / "quotient_check"
    subprocess.run(["gcc", "-O2", "-mfma", "-fopenmp", "-ffp-contract=off",
                    os.path.join(HERE, "host", "quotient_check.c"), "-o", str(exe), "-lm"],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert out.stdout.strip() == "0", out.stdout + out.stderr
