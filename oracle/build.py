"""Build the CPU oracle library (oracle/liboracle.so) with gcc.

Test infrastructure: the oracle is the independent checker of the HIP path.
Flags: -O2, no FP contraction (every fp32/fp64 operation rounds on its own),
no fast-math, OpenMP only over independent rows.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "bitlinear_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
         "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(extra_flags=(), out=LIB, quiet=False):
    """Compile the oracle. extra_flags lets tests build planted-mistake variants."""
    cmd = ["gcc", *FLAGS, *extra_flags, SRC, "-o", out + ".tmp", "-lm"]
    if not quiet:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(sys.argv[1:])
