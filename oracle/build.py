"""Builds liboracle.so from gs_oracle.cpp with the host compiler (test infrastructure only).

Contraction is off so that every fp32 expression rounds in the order it is written; the only
fused multiply-adds are the explicit std::fma calls of the D1 exp/log.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gs_oracle.cpp")
OUT = os.path.join(HERE, "liboracle.so")

FLAGS = ["-O2", "-std=c++17", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(verbose: bool = False) -> str:
    cmd = ["g++", *FLAGS, "-o", OUT + ".tmp", SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
