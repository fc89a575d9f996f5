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


def build_sanitized(out: str, verbose: bool = False, src: str = SRC) -> str:
    """The same source with AddressSanitizer and UndefinedBehaviorSanitizer, every report
    fatal, for the sanitizer test (loaded through ORACLE_LIB with the runtimes preloaded)."""
    cc = os.environ.get("ORACLE_CC", "gcc")
    cmd = [cc, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", out, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
