"""Build the CPU oracle (test infrastructure) as oracle/libthrift_oracle.so.

Plain C11, fp64, no fast-math and no floating-point contraction, so every
rounding in the oracle is the one its source writes.  OpenMP only spreads
independent query rows over the host cores.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libthrift_oracle.so")


def build(verbose: bool = False, src: str = None, out: str = None) -> str:
    src = src or os.path.join(HERE, "thrift_oracle.c")
    lib = out or LIB
    tmp = lib + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-I", HERE, "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
