"""Build the CPU oracle library (plain C, gcc, OpenMP).

Test infrastructure: the library built here is loaded only by the tests, the
smoke check and the CPU-baseline leg of the benchmark.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lattn_oracle.c")
LIB = os.path.join(HERE, "liblattn_oracle.so")


def build(src: str = SRC, out: str = LIB, extra_flags: list[str] | None = None) -> str:
    """Compile ``src`` into the shared library ``out`` and return its path."""
    cmd = ["gcc", "-std=c11", "-O3", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           src, "-o", out + ".tmp", "-lm"] + list(extra_flags or [])
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
