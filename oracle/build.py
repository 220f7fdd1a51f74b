"""Build the CPU oracle (test infrastructure): oracle/libfq_oracle.so.

Plain C, -O2 without fast-math or FP contraction, so that every float
expression in fq_oracle.c is one IEEE binary32 operation rounded to nearest.
OpenMP only splits independent rows across threads.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fq_oracle.c")
LIB = os.path.join(HERE, "libfq_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-std=c11", "-O2", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
        "-Wall", "-Wextra",
        SRC, "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def ensure_built() -> str:
    """Build only if the library is missing or older than its source."""
    if (not os.path.exists(LIB)
            or os.path.getmtime(LIB) < os.path.getmtime(SRC)):
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
