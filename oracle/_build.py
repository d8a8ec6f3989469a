"""Compile the C oracle into ``oracle/liboracle.so`` (gcc, no GPU code).

Flags keep the arithmetic as written: no FMA contraction, no fast-math.
"""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build_oracle(verbose: bool = False) -> str:
    cmd = [
        "gcc",
        "-std=c99",
        "-O2",
        "-fPIC",
        "-shared",
        "-ffp-contract=off",
        "-fno-fast-math",
        "-D_GNU_SOURCE",
        "-Wall",
        "-fopenmp",
        "-o",
        LIB + ".tmp",
        SRC,
        "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build_oracle(verbose=True))
