"""Builds _build/libzero_dp_hostcheck.so: the library's host translation
units (planner, memory model, argument validation and the C entry points)
compiled for the CPU with the address and undefined-behaviour sanitizers,
linked against launchers that report "no device" for every launch
(csrc/zero_dp_nodevice.cpp).  No device code is compiled or linked.

    python -m zero_partitioned_mixed_buffer_amd.hostcheck_build

The host-side tests then run against it (the binding loads the library
named by ZERO_DP_LIBRARY) with the sanitizer runtime preloaded.
"""
from __future__ import annotations

import os
import subprocess
import sys

from .build_lib import BUILD, CSRC, HOST_FLAGS, HOST_SOURCES, INCLUDE

LIB = os.path.join(BUILD, "libzero_dp_hostcheck.so")
FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def runtime() -> str:
    """Path of the address-sanitizer runtime that must be preloaded."""
    return subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [os.path.join(CSRC, f) for f in (*HOST_SOURCES, "zero_dp_nodevice.cpp")]
    tmp = LIB + ".tmp"
    cmd = ["g++", *HOST_FLAGS, *FLAGS, "-I", INCLUDE, "-shared", *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host-check build failed ({r.returncode}):\n{r.stdout}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
