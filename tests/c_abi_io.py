"""Input and output files of tests/c_abi/zero_step_file (the plain C
consumer of the ABI): the layout its header comment states."""
from __future__ import annotations

import os
import struct
import subprocess

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi", "zero_step_file")


def ensure_built() -> str:
    """The program as build() left it; built here (gcc, about a second) only
    when it is missing."""
    if not os.path.exists(EXE):
        from tests.c_abi import build_c_abi
        build_c_abi.build()
    return EXE


def write_input(path, master0, ag0, ag_off, nd, L, hp, step_slices):
    n = master0.size
    with open(path, "wb") as f:
        f.write(b"ZDPSTEP1")
        f.write(struct.pack("<qqqii", n, ag0.size, ag_off, nd, len(step_slices)))
        f.write(struct.pack("<6d", L, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"]))
        f.write(np.ascontiguousarray(master0, dtype="<f4").tobytes())
        f.write(np.ascontiguousarray(ag0, dtype="<u2").tobytes())
        for sl in step_slices:
            assert sl.shape == (nd, n) and sl.dtype == np.float16
            f.write(np.ascontiguousarray(sl).view("<u2").tobytes())


def read_output(path, n, ag_len, steps):
    out = []
    with open(path, "rb") as f:
        assert f.read(8) == b"ZDPOUT01"
        for _ in range(steps):
            cur, t, ovf, _pad = struct.unpack("<4i", f.read(16))
            sumsq, skipped = struct.unpack("<dq", f.read(16))
            st = np.frombuffer(f.read(12 * n), dtype="<f4").reshape(3, n)
            ag = np.frombuffer(f.read(2 * ag_len), dtype="<u2")
            out.append(dict(cur=cur, t=t, overflow=ovf, sumsq=sumsq, skipped=skipped,
                            p=st[0], m=st[1], v=st[2], ag=ag))
        assert f.read(1) == b""
    return out


def run(in_path, out_path, mode="step", timeout=120):
    return subprocess.run([EXE, in_path, out_path, mode], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                          text=True, timeout=timeout)
