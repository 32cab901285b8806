"""Host AddressSanitizer + UndefinedBehaviorSanitizer runs (CPU only).

* The CPU oracle (oracle/svdq_oracle.c), compiled with gcc into a driver
  that calls every exported function on exact-size heap buffers with the
  edge values of the parity tests.
* The C ABI layer (csrc/svdq_abi.hip, host code only), compiled with g++
  against stand-ins for the kernels' launchers and the HIP device query, and
  driven through every entry point of include/svdq.h: valid calls must reach
  the right launcher, invalid ones must be rejected before any launch.

Both are built with -fno-sanitize-recover=all, so any report aborts the
program."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "host_sanitize")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, cwd):
    res = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=ENV, timeout=300)
    return res.returncode, res.stdout + res.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    rc, out = _run(["gcc", "-std=c11", "-ffp-contract=off", *SAN, "-o", exe,
                    os.path.join(SRC, "oracle_driver.c"), "-lm"], str(tmp_path))
    assert rc == 0, out
    rc, out = _run([exe], str(tmp_path))
    assert rc == 0 and "oracle sanitize ok" in out, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"),
                    reason="needs g++ and the HIP headers")
def test_abi_host_checks_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_driver")
    srcs = [os.path.join(SRC, f) for f in ("abi_host.cpp", "hip_stubs.cpp", "abi_driver.cpp")]
    rc, out = _run(["g++", "-std=c++20", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", *SAN, "-o", exe, *srcs],
                   str(tmp_path))
    assert rc == 0, out
    rc, out = _run([exe], str(tmp_path))
    assert rc == 0 and "abi sanitize ok" in out, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
