"""Build the fp64 CPU oracle (test infrastructure): plain C with OpenMP, no BLAS."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB_PATH = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra"]


def compile_oracle(src: str, out: str, extra: list[str] | None = None) -> None:
    """Compile one oracle source file into a shared library (used for the
    in-tree build and for test-only variants)."""
    cmd = ["gcc", *CFLAGS, *(extra or []), src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(out + ".tmp", out)


def build() -> str:
    compile_oracle(SRC, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
