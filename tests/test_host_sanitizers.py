"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

A copy of libra.so is built with both sanitizers on the host pass only, and
the CPU ABI tests (every entry point's argument validation, the size-limit
checks at their boundaries, the error strings) run against it in a child
process that preloads the ASan runtime. Any heap or stack overflow, use after
free, signed overflow in the size arithmetic or other undefined behaviour
aborts that process. No GPU is used: every call returns before a launch."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(900)
def test_abi_validation_under_host_asan_and_ubsan():
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc is not available")
    bhs = pytest.importorskip("ring_attention_ra_amd.build_host_sanitized")
    lib = bhs.build()
    runtime = bhs.asan_runtime()

    # the host code really is instrumented
    undefined = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True,
                               check=True).stdout
    assert "__asan_report_" in undefined and "__ubsan_handle_" in undefined

    env = dict(os.environ)
    env.update(RA_LIB=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join("tests", "test_abi.py"),
                          "-m", "not gpu", "-q", "-x", "-p", "no:cacheprovider"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
