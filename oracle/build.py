"""Build the C oracle into oracle/liboracle.so (host code only, gcc).

Test infrastructure: the GPU library neither builds nor links this.
Flags: no fast-math and no FMA contraction, so every float operation in the
oracle is a single IEEE-754 binary32 operation rounded to nearest even.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gmmfr_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = [
    "-O3", "-mavx2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
    "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
