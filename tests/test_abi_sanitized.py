"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).  The library is rebuilt with both sanitizers on its host code
(device code as usual; no kernel runs here) and tests/test_abi.py -- every
entry point's validation: null pointers, bad sizes and strides including
strides at and beyond the 2^31 bound, misalignment, overlapping buffers,
workspace sizing -- runs against it in a child process with the sanitizer
runtime preloaded.  Any sanitizer report aborts the child and fails this
test."""

import os
import subprocess
import sys

import pytest

from fp8_w8a8_dynamic_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(900)
def test_abi_suite_clean_under_asan_and_ubsan():
    lib = build.build_sanitized()
    env = dict(os.environ)
    env.update({
        "FP8W8A8_ABI_TEST_LIBRARY": lib,
        "LD_PRELOAD": build.sanitizer_runtime(),
        # Python itself is not instrumented: leaks at exit and the preload
        # order are not findings about this library.
        "ASAN_OPTIONS": "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
    })
    res = subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_abi.py")],
        env=env, capture_output=True, text=True, timeout=800, cwd=ROOT)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in res.stdout
