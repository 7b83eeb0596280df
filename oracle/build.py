"""Compile the CPU oracle (plain C, gcc, OpenMP) into oracle/libskoracle.so.

Test infrastructure: the library is loaded only by the test suite, the smoke
check and the CPU-baseline leg of the benchmark.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "skoracle.c")
OUT = os.path.join(HERE, "libskoracle.so")


def build(verbose: bool = False) -> str:
    # -ffp-contract=off: no fused multiply-add, every product and sum is a
    # separately rounded fp64 operation.
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", OUT + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
