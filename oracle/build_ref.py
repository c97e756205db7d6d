"""Builds the plain C++ oracle (h3_ref.cpp) into oracle/libh3ref.so with g++.

Test infrastructure: the tests, the smoke check and the benchmark's CPU
baseline load it; the product path never does.  No fused multiply-adds
(-ffp-contract=off) and no fast-math, so every fp32 operation rounds on its
own; x86-64-v3 (AVX2) lets the compiler process independent outputs together
on any host the library may run on.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "h3_ref.cpp")
LIB = os.path.join(HERE, "libh3ref.so")
FLAGS = ["-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
         "-std=c++17", "-Wall"]


def build():
    tmp = LIB + ".tmp"
    r = subprocess.run(["g++"] + FLAGS + [SRC, "-o", tmp, "-lm"], capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"oracle build failed (exit {r.returncode})")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print("built", build())
