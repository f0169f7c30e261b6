"""Builds the HIP library libmsamp.so for gfx950 with hipcc (in-tree)."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIB_DIR, "libmsamp.so")
SOURCES = [os.path.join(CSRC, "kernels.hip"), os.path.join(CSRC, "abi.hip")]
HEADERS = [os.path.join(CSRC, "codec.hpp"), os.path.join(CSRC, "device.hpp"), os.path.join(CSRC, "kernels.hpp"),
           os.path.join(INCLUDE, "msamp.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -ffp-contract=off: only explicit fmaf calls are fused (the AdamW operation
# order is part of the result). Packed FP32 instructions are disabled.
FLAGS = ["-std=c++17", "-O3", "-fPIC", "--offload-arch=" + ARCH, "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-command-line-argument", "-I" + INCLUDE, "-I" + CSRC]


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libmsamp.so. Always rebuilds."""
    os.makedirs(LIB_DIR, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(LIB_DIR, os.path.basename(src) + ".o")
        cmd = [HIPCC] + FLAGS + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd))
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
