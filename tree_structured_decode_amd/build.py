"""Builds libdeft.so in-tree with hipcc for gfx950.

    python -m tree_structured_decode_amd.build

The HIP translation unit is compiled with packed-FP32 instructions disabled;
the host planner is plain C++.  Outputs go to tree_structured_decode_amd/
(libdeft.so) and tree_structured_decode_amd/_build/ (objects).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdeft.so")

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    return os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    if verbose and (r.stdout or r.stderr):
        sys.stderr.write(r.stdout + r.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    inc = ["-I", INCLUDE, "-I", CSRC]
    att_o = os.path.join(BUILD, "deft_attention.o")
    plan_o = os.path.join(BUILD, "deft_plan.o")
    _run([hipcc, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, "deft_attention.hip"), "-o", att_o], verbose)
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", *inc, "-c",
          os.path.join(CSRC, "deft_plan.cpp"), "-o", plan_o], verbose)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", "--offload-arch=gfx950", att_o, plan_o, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
