"""Compile the CPU oracle (test infrastructure) into ``oracle/liboracle.so``.

Plain gcc, strict IEEE evaluation: no fused multiply-add contraction, no
fast-math, no host-specific instruction selection.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "skipln_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CMD = [
    "gcc",
    "-O2",
    "-std=c99",
    "-D_POSIX_C_SOURCE=200809L",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-Wall",
    "-Wextra",
    "-Werror",
    "-fPIC",
    "-shared",
    "-pthread",
    SRC,
    "-o",
]


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + f".tmp{os.getpid()}"
    subprocess.run(CMD + [tmp, "-lm"], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--if-stale" not in sys.argv))
