"""The C-ABI validation tests (tests/test_abi.py) run again against a build of
the library whose host code carries AddressSanitizer and
UndefinedBehaviorSanitizer (`python -m layer_backward_pass_amd._build
--sanitize`): every argument check, size limit and checking pass of every
entry point then runs under the sanitizers.  The build is refreshed when a
source is newer than it; the sanitizer runtime is preloaded into a child
Python (the interpreter itself is not instrumented), so leak detection is off.
"""
import glob
import os
import subprocess
import sys

import pytest

from layer_backward_pass_amd import _build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _stale():
    if not os.path.exists(B.SAN_LIB):
        return True
    t = os.path.getmtime(B.SAN_LIB)
    srcs = glob.glob(os.path.join(B.CSRC, "*")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
    return any(os.path.getmtime(p) > t for p in srcs)


@pytest.mark.timeout(900)
def test_abi_tests_under_host_sanitizers():
    rt = B.sanitizer_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    if _stale():
        B.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=rt, LORABWD_LIB=B.SAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in out and "ERROR: AddressSanitizer" not in out and "runtime error" not in out
