"""The host-side argument validation of every C-ABI call under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU: the library is
built with both sanitizers on its host code, and the boundary tests (every
call rejecting NULL, misaligned, short or inconsistent arguments before any
launch) run against that build in a child process with the sanitizer runtime
preloaded.  Any out-of-bounds access, use after free or undefined behaviour
in the validation layer aborts the child and fails this test."""

import os
import subprocess
import sys

import pytest

from megatron_tensor_transformer_02_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(900)
def test_boundary_checks_under_asan_and_ubsan():
    lib = build.build(sanitize=True)
    runtime = build.asan_runtime()
    assert os.path.exists(runtime), runtime
    env = dict(os.environ, MP_LIB=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_boundary.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out
