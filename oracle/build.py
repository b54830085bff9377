"""Compile the CPU oracle (plain C) into oracle/liboracle.so with gcc.

Test infrastructure only: the product library never links or loads it.
Floating-point contraction and fast-math are off so every operation is the
IEEE operation the source spells out.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nf4_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [
        "gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp",
        "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
        "-Wall", "-Wextra", "-o", tmp, SRC, "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
