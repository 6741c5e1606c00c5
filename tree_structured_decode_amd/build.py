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
SANITIZED_LIB = os.path.join(BUILD, "libdeft_host_sanitized.so")
BENCH_LIB = os.path.join(PKG, "libdeft_bench.so")

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
    # the streaming-read calibration kernel the benchmark times
    bench_o = os.path.join(BUILD, "deft_bench.o")
    _run([hipcc, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, "deft_bench.hip"), "-o", bench_o], verbose)
    tmp = BENCH_LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", "--offload-arch=gfx950", bench_o, "-o", tmp], verbose)
    os.replace(tmp, BENCH_LIB)
    return LIB


def build_planner_sanitized(verbose: bool = False) -> str:
    """The host planner alone (deft_plan.cpp plus host-only stand-ins for the
    HIP entry points), built with AddressSanitizer and UndefinedBehavior-
    Sanitizer for the CPU test suite; load it with libasan preloaded."""
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", INCLUDE, "-I", CSRC]
    tmp = SANITIZED_LIB + ".tmp"
    _run(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-fPIC", "-shared", "-Wall", *inc,
          os.path.join(CSRC, "deft_plan.cpp"), os.path.join(CSRC, "deft_host_only.cpp"), "-o", tmp], verbose)
    os.replace(tmp, SANITIZED_LIB)
    return SANITIZED_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
