"""The plain C consumer of the ABI (tests/c_abi/zero_step_file) builds with
gcc against include/zero_dp.h and the in-tree library, and rejects bad
usage and malformed input before it makes any HIP call (no GPU needed)."""
import struct
import subprocess

import pytest

from c_abi_io import ensure_built

pytest.importorskip("zero_partitioned_mixed_buffer_amd.binding")


@pytest.fixture(scope="module")
def exe():
    return ensure_built()


def _run(*args):
    return subprocess.run(list(args), stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=60)


def test_usage_errors(exe, tmp_path):
    r = _run(exe)
    assert r.returncode == 2 and "usage" in r.stdout
    r = _run(exe, "a", "b", "sideways")
    assert r.returncode == 2 and "usage" in r.stdout
    r = _run(exe, str(tmp_path / "missing.bin"), str(tmp_path / "out.bin"))
    assert r.returncode == 2 and "cannot open" in r.stdout


@pytest.mark.parametrize("header,why", [
    (b"ZDPSTEPX" + struct.pack("<qqqii", 8, 8, 0, 1, 1) + struct.pack("<6d", 1, 1e-3, 0.9, 0.999, 1e-8, 0), "magic"),
    (b"ZDPSTEP1" + struct.pack("<qqqii", 8, 4, 0, 1, 1) + struct.pack("<6d", 1, 1e-3, 0.9, 0.999, 1e-8, 0),
     "window past the buffer"),
    (b"ZDPSTEP1" + struct.pack("<qqqii", 8, 8, 0, 0, 1) + struct.pack("<6d", 1, 1e-3, 0.9, 0.999, 1e-8, 0), "nd 0"),
    (b"ZDPSTEP1" + struct.pack("<qqqii", -8, 8, 0, 1, 1) + struct.pack("<6d", 1, 1e-3, 0.9, 0.999, 1e-8, 0),
     "negative n"),
    (b"ZDPSTEP1" + struct.pack("<qqq", 8, 8, 0), "truncated"),
])
def test_malformed_input_is_rejected(exe, tmp_path, header, why):
    fin = tmp_path / "in.bin"
    fin.write_bytes(header)
    r = _run(exe, str(fin), str(tmp_path / "out.bin"))
    assert r.returncode == 2, (why, r.stdout)
    assert "bad input header" in r.stdout or "input ends early" in r.stdout, (why, r.stdout)
