"""Compile the CPU oracle (test infrastructure) into oracle/liboracle.so.

Plain gcc, -O2, no floating-point contraction and no fast-math, so every
binary32/binary64 operation in oracle.c is the IEEE operation it is written as.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
SRC = [os.path.join(HERE, "oracle.c")]
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-fno-finite-math-only", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, *SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
