"""Compile the oracle's C part (test infrastructure) into oracle/liboracle.so."""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CMD = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
       "-fPIC", "-shared", "-o", LIB, SRC, "-lm"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = CMD[:-3] + [tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
