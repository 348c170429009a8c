"""Build the CPU oracle (plain C, gcc) into oracle/liboracle.so.

The oracle is test infrastructure; building it is part of the build check so
that the tests can use it, and nothing on the product path loads it.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dflash2_oracle.c")
OUT = os.path.join(HERE, "liboracle.so")

# No fast-math, no contraction: the path search is defined on float
# additions, and the double sums must not be reassociated.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
          "-ffp-contract=off", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", OUT + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
