"""Compile the fp64 oracle (test infrastructure only) into a shared library.

    python -m oracle.build          # writes oracle/liboracle.so
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-fPIC", "-shared", "-std=c99", "-fno-fast-math",
          "-ffp-contract=off", "-fopenmp", "-Wall", "-Wextra"]


def compile_oracle(src: str = SRC, out: str = LIB, extra=()) -> str:
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def ensure_built() -> str:
    """Build if the library is missing or older than its source."""
    if (not os.path.exists(LIB)) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        compile_oracle()
    return LIB


if __name__ == "__main__":
    print(compile_oracle(), file=sys.stderr)
