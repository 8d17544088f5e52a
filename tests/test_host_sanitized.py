"""The library's host code under the address and undefined-behaviour
sanitizers (no GPU): the host translation units are built alone with ASan
and UBSan (zero_partitioned_mixed_buffer_amd/hostcheck_build.py, launchers
that report "no device"), and the host-side ABI tests run against that
build in a child process with the sanitizer runtime preloaded.  Any
out-of-bounds access, use after free, signed overflow, misaligned access or
other undefined behaviour in the planner, the memory model or the argument
validation of any entry point aborts the child and fails this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(600)
def test_host_abi_tests_under_asan_ubsan():
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("LD_PRELOAD is already set by the environment; the sanitizer runtime must come first")
    sys.path.insert(0, ROOT)
    from zero_partitioned_mixed_buffer_amd import hostcheck_build
    lib = hostcheck_build.build()
    env = dict(os.environ, LD_PRELOAD=hostcheck_build.runtime(), ZERO_DP_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("PYTEST_ADDOPTS", None)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=540)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert " passed" in r.stdout and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out


def test_hostcheck_build_has_no_device_code():
    """The sanitizer build links the no-device launchers: a call that passes
    validation returns ZERO_EHIP with hipErrorNoDevice, computing nothing."""
    import ctypes as C
    sys.path.insert(0, ROOT)
    from zero_partitioned_mixed_buffer_amd import hostcheck_build
    lib = hostcheck_build.build()
    r = subprocess.run(["nm", "-D", "--defined-only", lib], capture_output=True, text=True, check=True)
    assert "hipLaunchKernel" not in r.stdout and "__hip" not in r.stdout
    assert "zero_adam_step_noalloc" in r.stdout and "zero_gather_params" in r.stdout
