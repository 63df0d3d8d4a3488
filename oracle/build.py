"""Builds the CPU oracle library oracle/liboracle.so with gcc.

Test infrastructure only (see oracle/__init__.py).  The flags keep every
binary32 operation of the quantizer a single correctly rounded IEEE operation:
no floating-point contraction, no fast-math.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
        "-fopenmp", "-shared", "-fPIC", "-Wall", "-Wextra",
        os.path.join(HERE, "kivi_oracle.c"), "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
