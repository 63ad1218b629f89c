"""Compile the oracle's C part (test infrastructure) into oracle/liboracle.so.

    python -m oracle.build [-v] [--sanitize]

--sanitize builds oracle/liboracle_san.so with clang, AddressSanitizer and
UndefinedBehaviorSanitizer (for a test process started with clang's ASan
runtime preloaded; tests/conftest.py picks it up from ORACLE_TEST_LIB).
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
SAN_LIB = os.path.join(HERE, "liboracle_san.so")

CMD = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
       "-fPIC", "-shared", "-o", LIB, SRC, "-lm"]
SAN_CC = "/opt/rocm/llvm/bin/clang"
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    lib = SAN_LIB if sanitize else LIB
    tmp = lib + ".tmp"
    cc = [SAN_CC] if sanitize else CMD[:1]
    cmd = cc + CMD[1:-4] + (SAN_FLAGS if sanitize else []) + ["-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
