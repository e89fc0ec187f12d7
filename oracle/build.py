"""Build the CPU oracle (plain C, gcc) into ``oracle/liboracle.so``.

Flags: ``-O3 -fopenmp -ffp-contract=off`` and no fast-math, so every float
operation is the IEEE operation written in the source (``fmaf`` only where the
source calls it).
"""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [
        "gcc", "-std=c11", "-O3", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
        "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unused-parameter", SRC, "-o", tmp, "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
