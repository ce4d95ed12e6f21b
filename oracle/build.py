"""Builds liboracle.so from gs_oracle.cpp with the host compiler (test infrastructure only).

Contraction is off so that every fp32 expression rounds in the order it is written; the only
fused multiply-adds are the explicit std::fma calls of the D1 exp/log.

``python oracle/build.py --debug`` builds liboracle_asan.so instead: -O1 -g with AddressSanitizer
and UndefinedBehaviorSanitizer (host code only). The oracle loads it when GS_ORACLE_LIB names it;
the interpreter then needs the sanitizer runtime preloaded, e.g.
    GS_ORACLE_LIB=oracle/liboracle_asan.so LD_PRELOAD=$(g++ -print-file-name=libasan.so) \
    ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=print_stacktrace=1 python -m pytest tests -m "not gpu"
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gs_oracle.cpp")
OUT = os.path.join(HERE, "liboracle.so")
OUT_DEBUG = os.path.join(HERE, "liboracle_asan.so")

FLAGS = ["-O2", "-std=c++17", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]
DEBUG_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-std=c++17", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(verbose: bool = False, debug: bool = False) -> str:
    out = OUT_DEBUG if debug else OUT
    cmd = ["g++", *(DEBUG_FLAGS if debug else FLAGS), "-o", out + ".tmp", SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, debug="--debug" in sys.argv))
    sys.exit(0)
