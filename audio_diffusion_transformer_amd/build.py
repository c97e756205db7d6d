"""Build steps: the synthetic-input generator (gcc) and the HIP library (hipcc, gfx950).

Everything is built in-tree so that the shared objects travel with the source tree.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_H3 = os.path.join(PKG, "libh3.so")
LIB_SYNTH = os.path.join(PKG, "synth", "libh3synth.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    # keep the compiler from forming packed fp32 VALU ops in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build failed: {' '.join(cmd[:3])} ... (exit {r.returncode})")
    return r


def build_synth():
    src = os.path.join(PKG, "synth", "synth.c")
    tmp = LIB_SYNTH + ".tmp"
    _run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", src, "-o", tmp, "-lm"])
    os.replace(tmp, LIB_SYNTH)
    return LIB_SYNTH


def hip_sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def build_hip(extra=()):
    tmp = LIB_H3 + ".tmp"
    cmd = [HIPCC] + HIP_FLAGS + list(extra) + ["-I", INCLUDE, "-I", CSRC] + hip_sources() + ["-o", tmp]
    r = _run(cmd)
    warn = [l for l in (r.stdout + r.stderr).splitlines()
            if "warning" in l and "packed-fp32-ops" not in l]
    if warn:
        sys.stderr.write("\n".join(warn) + "\n")
    os.replace(tmp, LIB_H3)
    return LIB_H3


def build_all():
    build_synth()
    build_hip()


if __name__ == "__main__":
    build_all()
    print("built", LIB_SYNTH, LIB_H3)
