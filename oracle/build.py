"""Build the FP64 CPU oracle (test infrastructure only) with gcc.

Produces ``oracle/libgdn2_oracle.so`` next to the C source.  Plain ``-O2``
with no fast-math and no FMA contraction, so the oracle's rounding is that of
the written FP64 expressions.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn2_oracle.c")
LIB = os.path.join(HERE, "libgdn2_oracle.so")


def compile_oracle(src: str = SRC, out: str = LIB, extra_flags: list[str] | None = None) -> str:
    """Compile an oracle source file into a shared library and return its path."""
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
        "-o", out + ".tmp", src, "-lm",
    ]
    if extra_flags:
        cmd[1:1] = list(extra_flags)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def needs_build(src: str = SRC, out: str = LIB) -> bool:
    return (not os.path.exists(out)) or os.path.getmtime(out) < os.path.getmtime(src)


if __name__ == "__main__":
    print(compile_oracle(*sys.argv[1:3]))
