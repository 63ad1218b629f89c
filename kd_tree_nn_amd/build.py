"""Compile libkdnn.so (HIP for gfx950 + host C++) in-tree.

    python -m kd_tree_nn_amd.build [-v] [--resource-usage]

Every source is recompiled on each call.  Floating-point flags: no FP
contraction (-ffp-contract=off) and no fast-math, so the fp32 distance and
the fp64 transform are rounded operation by operation; packed fp32
instructions are disabled for device code.
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


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [cc, "-c", path, "-o", obj] + common_flags()
        if src.endswith(".hip"):
            cmd += device_flags()
            if resource_usage:
                cmd += ["-Rpass-analysis=kernel-resource-usage"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv, resource_usage="--resource-usage" in sys.argv)
    print(LIB)
