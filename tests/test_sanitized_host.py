"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The planner, every argument check and the dispatch's host paths run in the
ABI tests (no GPU needed: every call there is refused or planned before any
device work). Here they run again against a build of the library whose host
code is instrumented with both sanitizers, in a child process with the
sanitizer runtime preloaded; any report fails the test.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(900)
def test_abi_tests_pass_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, os.path.join(ROOT, "lm_head_projection_token_amd"))
    try:
        import build_sanitized as bs
    finally:
        sys.path.pop(0)
    lib = bs.build_host_sanitized(str(tmp_path))
    env = dict(os.environ, FLL_LIBRARY=lib, LD_PRELOAD=bs.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # the child really runs the instrumented library under the runtime
    probe = subprocess.run(
        [sys.executable, "-c",
         "import ctypes, lm_head_projection_token_amd as f; "
         f"assert f.LIB_PATH == {lib!r}; "
         "ctypes.CDLL(None).__asan_init; "
         "print(f.fll_version())"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-3000:]
    res = subprocess.run(
        [sys.executable, "-m", "pytest", "tests/test_abi.py", "-q", "-x",
         "-p", "no:cacheprovider"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in res.stdout
