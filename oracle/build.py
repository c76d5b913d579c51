"""Build the CPU oracle (test infrastructure only) into oracle/liboracle.so.

Strict IEEE double arithmetic: no -ffast-math, no FMA contraction, so every
operation rounds exactly as written in oracle.c.  OpenMP is enabled for the
token loops of the router and the combine, which run on one thread unless
oracle.set_threads() asks for more (the benchmark's CPU baseline does).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", SRC, "-lm", "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
