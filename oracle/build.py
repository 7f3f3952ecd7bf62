"""Build the CPU oracle (test infrastructure) as oracle/liboracle.so with gcc.

IEEE fp32 semantics: no fast-math, no FMA contraction, SSE math on x86-64.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c99", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
          "-fopenmp", "-Wall", "-Wextra"]


def build(extra_flags=None, out=LIB) -> str:
    src = os.path.join(HERE, "oracle.c")
    cmd = ["gcc", *CFLAGS, *(extra_flags or []), "-shared", src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1:]))
