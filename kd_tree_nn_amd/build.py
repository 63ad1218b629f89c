"""Compile libkdnn.so (HIP for gfx950 + host C++) in-tree.

    python -m kd_tree_nn_amd.build [-v] [--resource-usage] [--sanitize]

Every source is recompiled on each call.  Floating-point flags: no FP
contraction (-ffp-contract=off) and no fast-math, so the fp32 distance and
the fp64 transform are rounded operation by operation; packed fp32
instructions are disabled for device code.

--sanitize builds libkdnn_san.so instead: the host code of every source
(builder, C ABI, host rigid solve, kernel launchers) instrumented with
AddressSanitizer and UndefinedBehaviorSanitizer; device code is built as
usual.  The sanitizer runtime is not linked in: load the library into a
process started with clang's ASan runtime preloaded (tests/conftest.py
picks the library named by KDNN_TEST_LIB).
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkdnn.so")
SAN_LIB = os.path.join(HERE, "libkdnn_san.so")
ARCH = "gfx950"

SOURCES = ["kernels.hip", "voxel.hip", "roofline.hip", "noalloc.hip", "builder.cpp",
           "procrustes.cpp", "capi.cpp"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math",
            "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def device_flags():
    return [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sanitize_flags():
    """ASan + UBSan for host code only (each flag scoped to the host pass)."""
    out = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
              "-fno-omit-frame-pointer", "-g"):
        out += ["-Xarch_host", f]
    return out


def build(verbose: bool = False, resource_usage: bool = False, sanitize: bool = False) -> str:
    bdir = BUILD + ("_san" if sanitize else "")
    lib = SAN_LIB if sanitize else LIB
    os.makedirs(bdir, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, "-c", path, "-o", obj] + common_flags()
        if src.endswith(".hip"):
            cmd += device_flags()
            if resource_usage:
                cmd += ["-Rpass-analysis=kernel-resource-usage"]
        if sanitize:
            cmd += sanitize_flags()
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = lib + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, resource_usage="--resource-usage" in sys.argv,
                sanitize="--sanitize" in sys.argv))
