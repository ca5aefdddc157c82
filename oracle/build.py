"""Compile the CPU oracle (test infrastructure) into oracle/liboracle.so."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "bitlinear_oracle.c")
OUT = os.path.join(HERE, "liboracle.so")
# No fast-math, no FMA contraction: every float/double operation in the source is
# one IEEE operation, in the order written.
FLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp"
    cmd = ["gcc", *FLAGS, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
