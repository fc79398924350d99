"""Compile the CPU oracle (``oracle.c``) into ``liboracle.so`` with gcc.

Test infrastructure: the oracle is used only by the tests, the smoke check
and the bench's CPU baseline leg.  Building it is not using it."""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    # Portable x86-64 code (no -march=native: the library may run on another
    # host); fp contraction off so every fp32 step rounds as written.
    cmd = ["gcc", "-O3", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
