"""Builds tests/c_abi/zero_step_file, a plain C program that drives owned-shard
steps through include/zero_dp.h alone, with gcc: linked against the in-tree
libzero_dp.so (found at run time next to the package, relative to the
program) and the HIP runtime it takes device memory from."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "zero_step_file.c")
EXE = os.path.join(HERE, "zero_step_file")
ROCM = "/opt/rocm"


def build(verbose: bool = False) -> str:
    pkg = os.path.join(ROOT, "zero_partitioned_mixed_buffer_amd")
    if not os.path.exists(os.path.join(pkg, "libzero_dp.so")):
        raise RuntimeError("libzero_dp.so is not built; build the library first")
    tmp = EXE + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC, "-o", tmp,
           "-L", pkg, "-lzero_dp", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../zero_partitioned_mixed_buffer_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C consumer build failed ({r.returncode}):\n{r.stdout}")
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
