"""Build the CPU oracle (test infrastructure) into oracle/liboracle.so with gcc.

Plain C99, -O2, no intrinsics, no floating-point contraction, OpenMP over output elements.  Run as a script or via build().
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qmm_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-Wall", "-Wextra", "-fopenmp", "-fPIC", "-shared",
           SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
