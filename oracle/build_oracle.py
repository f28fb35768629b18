"""Builds the CPU oracle (test infrastructure only) into oracle/libmoe_oracle.so.

The oracle is plain C compiled with gcc; it shares no source with the GPU path.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "libmoe_oracle.so")


def build(verbose: bool = False) -> str:
    # -O3 without -march=native: the built library travels to other hosts; with
    # -std=c99 gcc contracts no multiply-adds and reassociates no sums, so the
    # arithmetic is the source's, operation for operation
    cmd = ["gcc", "-O3", "-std=c99", "-fPIC", "-shared", "-fopenmp",
           "-Wall", "-Wno-unknown-pragmas", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
