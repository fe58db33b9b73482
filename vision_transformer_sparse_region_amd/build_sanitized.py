"""Build libbra_asan.so: the library with its host code under AddressSanitizer
and UndefinedBehaviorSanitizer (device code as in the product build).

    python -m vision_transformer_sparse_region_amd.build_sanitized

Used by the CPU test that runs the ABI tests against it (tests/test_sanitized_abi.py);
the GPU path never loads it.  The sanitizer flags reach only the host compilation.
"""
from __future__ import annotations

import glob
import os
import sys

from vision_transformer_sparse_region_amd.build import PKG, build_library

ASAN_LIB_PATH = os.path.join(PKG, "libbra_asan.so")
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime the sanitized library links against
    (preloaded into an uninstrumented Python)."""
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise FileNotFoundError("clang AddressSanitizer runtime not found under /opt/rocm/lib/llvm")
    return hits[-1]


def build_sanitized(out: str = ASAN_LIB_PATH, verbose: bool = False) -> str:
    return build_library(out, extra_flags=HOST_SANITIZE, link_flags=HOST_SANITIZE,
                         verbose=verbose)


if __name__ == "__main__":
    print(build_sanitized(verbose=True), file=sys.stderr)
