"""The ABI validation tests (tests/test_abi.py) rerun against a build of the library
whose host code in api.hip -- argument validation, overflow checks, the device
check and schedule choice -- is instrumented with AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU, no compute calls).  Any sanitizer report aborts
the child process and fails this test."""

import os
import subprocess
import sys

import pytest

from fp8_block_scaled_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_abi_validation_under_host_asan_and_ubsan():
    lib = build.SAN_LIB
    if not os.path.exists(lib):
        build.build_sanitized_abi()
    out = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in out and "__ubsan_handle" in out, "the library is not instrumented"
    env = dict(os.environ)
    env.update({
        "FP8BS_LIBRARY": lib,
        "LD_PRELOAD": build.sanitizer_runtime(),
        # CPython itself is not instrumented: leak reports would be its own.
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    code = ("import sys, pytest\n"
            "from fp8_block_scaled_amd import _lib\n"
            f"assert _lib.LIB_PATH == {lib!r}, _lib.LIB_PATH\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_abi.py']))\n")
    p = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert p.returncode == 0, p.stdout[-3000:] + p.stderr[-3000:]
    assert "passed" in p.stdout and "ERROR: AddressSanitizer" not in p.stderr
