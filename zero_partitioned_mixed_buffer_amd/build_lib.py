"""Builds libzero_dp.so in-tree for gfx950 with hipcc.

    python -m zero_partitioned_mixed_buffer_amd.build_lib [--asm]

The host translation units (planner, memory model, argument validation and
the C entry points) are compiled with g++, the HIP translation unit
(kernels and their launchers) with hipcc, and both are linked into one
shared library next to this file.  ``--asm`` also writes the gfx950
assembly of the kernels to _build/ for inspection.  (hostcheck_build.py
builds the host units alone under the sanitizers.)
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libzero_dp.so")
HOST_SOURCES = ("zero_dp_host.cpp", "zero_dp_calls.cpp")
# the step's kernels and launchers; the benchmark's calibration kernels
DEVICE_SOURCES = ("zero_dp_kernels.hip", "zero_dp_calib.hip")
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # float64 step arithmetic must not be contracted into FMAs
    "-ffp-contract=off",
    # no packed-fp32 instruction selection
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-ffp-contract=off"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    return r.stdout


def build(verbose: bool = False, asm: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    objs = []
    for src in HOST_SOURCES:
        o = os.path.join(BUILD, src.replace(".cpp", ".o"))
        _run(["g++", *HOST_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", o], verbose)
        objs.append(o)
    dev_objs = []
    for src in DEVICE_SOURCES:
        o = os.path.join(BUILD, src.replace(".hip", ".o"))
        _run([hipcc, *HIP_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", o], verbose)
        dev_objs.append(o)
    if asm:
        _run([hipcc, *HIP_FLAGS, "-I", INCLUDE, "--cuda-device-only", "-S",
              os.path.join(CSRC, "zero_dp_kernels.hip"), "-o", os.path.join(BUILD, "zero_dp_kernels.s")],
             verbose)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, *dev_objs, "-o", tmp,
          "-Wl,-rpath,/opt/rocm/lib"], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, asm="--asm" in sys.argv))
