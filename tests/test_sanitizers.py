"""AddressSanitizer and UndefinedBehaviorSanitizer over the host code (CPU only).

* The library's C-ABI host code (validation, planning, handle building,
  argument checks) built with g++ and both sanitizers, driven by
  tests/sanitize/host_driver.cpp over thousands of configurations, well-formed
  and malformed; the HIP runtime calls are host-memory stand-ins and the
  kernel launchers stubs, so no GPU code is built or run.
* The oracle built with gcc and both sanitizers, driven by
  tests/sanitize/oracle_driver.c over every feature at small sizes.
Any sanitizer finding aborts the driver (no recovery), failing the test."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-O1", "-g"]


def _run(cmd_build, exe):
    r = subprocess.run(cmd_build, capture_output=True, text=True)
    if r.returncode != 0:
        if "asan" in r.stderr.lower() or "sanitizer" in r.stderr.lower():
            pytest.skip("sanitizer runtime not available: " + r.stderr[-300:])
        raise AssertionError(r.stderr)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    out = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert out.returncode == 0, out.stdout[-2000:] + out.stderr[-4000:]
    return out.stdout


def test_host_code_under_sanitizers():
    gxx = shutil.which("g++")
    inc = "/opt/rocm/include"
    if not gxx or not os.path.exists(os.path.join(inc, "hip", "hip_runtime_api.h")):
        pytest.skip("g++ or the HIP headers not available")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "host_driver")
        out = _run([gxx, "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", inc, "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "quantized_recurrent_state_qstate_amd", "csrc"),
                    os.path.join(ROOT, "quantized_recurrent_state_qstate_amd", "csrc", "qstate_host.cpp"),
                    os.path.join(HERE, "host_driver.cpp"), "-o", exe], exe)
    assert "0 failed checks" in out, out


def test_oracle_under_sanitizers():
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not available")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_driver")
        out = _run([gcc, "-std=c11", *SAN, "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"),
                    os.path.join(ROOT, "oracle", "qs_oracle.c"), os.path.join(HERE, "oracle_driver.c"),
                    "-o", exe, "-lm"], exe)
    assert "0 failures" in out, out
