"""Build libbra.so in-tree with hipcc for gfx950.

    python -m vision_transformer_sparse_region_amd.build

The library is the product's compute path (HIP kernels + the C ABI of
include/bra.h).  Packed FP32 instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libbra.so")
SOURCES = [os.path.join(CSRC, n) for n in
           ("bra_pool.hip", "bra_route.hip", "bra_attend.hip", "bra_image.hip", "bra_small.hip",
             "bra_proj.hip", "bra_noalloc.hip", "bra_api.cpp")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
BUILD_TIMEOUT_S = 600  # a compile that runs longer is a code-size blow-up, not progress
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def build_library(out: str = LIB_PATH, extra_flags=(), verbose: bool = False,
                  link_flags=()) -> str:
    """Compile every source and link `out`; raises CalledProcessError on failure."""
    objs = []
    tag = os.path.splitext(os.path.basename(out))[0]
    for src in SOURCES:
        obj = os.path.join(CSRC, f"{os.path.basename(src)}.{tag}.o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC, *FLAGS, *extra_flags, *lang, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        subprocess.run(cmd, check=True, timeout=BUILD_TIMEOUT_S)
        objs.append(obj)
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_flags, *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True, timeout=BUILD_TIMEOUT_S)
    os.replace(tmp, out)
    for obj in objs:
        os.remove(obj)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True), file=sys.stderr)
