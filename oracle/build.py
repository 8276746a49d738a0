"""Compile the CPU oracle (plain C) into oracle/liboracle.so.

Test infrastructure only.  Flags keep the arithmetic exactly as written:
no FMA contraction, no fast-math reassociation.  -O3 with AVX2 lets the
compiler put the four rows a matvec walks side by side into one vector
register; each row's sum still runs sequentially in ascending index, so the
results are the same bits as a scalar build (a pin checks this).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "oracle.c")
    cmd = ["gcc", "-O3", "-mavx2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math",
           "-fopenmp", "-fPIC", "-shared", src, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def ensure_built() -> str:
    src = os.path.join(HERE, "oracle.c")
    hdr = os.path.join(HERE, "oracle.h")
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < max(os.path.getmtime(src), os.path.getmtime(hdr)):
        build()
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
