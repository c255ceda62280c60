"""Build the CPU oracle library with gcc (plain C, -O2, OpenMP over rows, no fast-math)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "gemv_oracle.c")
LIB_PATH = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror"]


def build(source: str = SOURCE, out: str = LIB_PATH, extra=()) -> str:
    """Compile `source` into the shared library `out` and return its path."""
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra, source, "-lm", "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
    sys.exit(0)
