"""Compile the CPU oracle into oracle/libcsa2_oracle.so with gcc.

Test infrastructure only.  The flags keep binary64 arithmetic exactly as
written: no fast-math, no fused multiply-add contraction, SSE2 (not x87).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csa2_oracle.c")
LIB = os.path.join(HERE, "libcsa2_oracle.so")

FLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fexcess-precision=standard",
         "-msse2", "-mfpmath=sse", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *FLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def ensure_built() -> str:
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
