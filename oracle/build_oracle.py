"""Build the fp64 CPU oracle (test infrastructure) with the host C compiler.

Produces ``oracle/liboracle_qdelta.so`` from ``oracle/qdelta_oracle.c``.  Plain
``gcc -O2 -fopenmp -ffp-contract=off``: no fused multiply-adds, so every product
and sum is a separately rounded fp64 operation.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qdelta_oracle.c")
LIB = os.path.join(HERE, "liboracle_qdelta.so")


def build(verbose: bool = False) -> str:
    cc = os.environ.get("ORACLE_CC", "gcc")
    cmd = [cc, "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
