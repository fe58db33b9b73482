"""Build liboracle.so from bra_oracle.c with the host C compiler.

Flags: -O2 -fopenmp -ffp-contract=off (a product is rounded before it is
added, as the plain loops are written), no fast-math.  TEST INFRASTRUCTURE.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "bra_oracle.c")
LIB_PATH = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build_oracle(src: str = SRC, out: str = LIB_PATH, extra_flags=()) -> str:
    """Compile `src` into the shared library `out`; returns `out`."""
    cc = os.environ.get("CC", "gcc")
    tmp = out + ".tmp"
    cmd = [cc, *CFLAGS, *extra_flags, "-I", HERE, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_oracle(), file=sys.stderr)
