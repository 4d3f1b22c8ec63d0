"""Builds the CPU oracle (test infrastructure) into oracle/liboracle.so with gcc.

Only tests/, the smoke check and the benchmark's CPU-baseline leg load the result.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "glu_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, src: str = SRC, lib: str = LIB) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", lib + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
