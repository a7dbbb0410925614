"""Builds the oracle library (liboracle_adahop.so) with gcc.

Test infrastructure only: the product path never loads this library.
-ffp-contract=off keeps every fp32/fp64 operation a separately rounded one.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle_adahop.so")


def build(verbose: bool = False, extra_flags=()) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-fopenmp", "-Wall", "-Wextra", *extra_flags,
           os.path.join(HERE, "adahop_ref.c"), "-o", LIB, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
