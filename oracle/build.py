"""Compile the CPU oracle (plain C, fp64, OpenMP) into oracle/libckoracle.so.

Test infrastructure: the oracle is built so that the test suite, the smoke
check and the benchmark's CPU-baseline leg can call it; the product never does.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ck_oracle.c")
LIB = os.path.join(HERE, "libckoracle.so")
# Same source evaluated in fp32: the method's fp32 rounding floor.
LIB_F32 = os.path.join(HERE, "libckoracle_f32.so")


# Integer fixed-point LIF forward (a second workload on the same graph class).
LIF_SRC = os.path.join(HERE, "lif_oracle.c")
LIF_LIB = os.path.join(HERE, "libliforacle.so")


def build(verbose: bool = False) -> str:
    for out, extra in ((LIB, []), (LIB_F32, ["-DOR_REAL=float"])):
        cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
               "-ffp-contract=off"] + extra + ["-o", out, SRC, "-lm"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-o", LIF_LIB, LIF_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
