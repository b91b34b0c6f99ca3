"""The C ABI's host validation under AddressSanitizer and UndefinedBehaviorSanitizer.

api.cpp is rebuilt by g++ with both sanitizers (host code only) and linked with the
ordinary kernel objects; the ABI host tests (every argument error of every call, the
descriptor layouts, the exports) then run against that library in a child process with
the ASan runtime preloaded. Any sanitizer report aborts the child and fails this test.
No GPU is used: every call in those tests fails validation before any HIP call.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ is needed for the host-sanitizer build")
def test_abi_host_checks_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from long_context_sparse_07_amd import sanitize
    lib = sanitize.build_sanitized()
    env = dict(os.environ)
    env.update(LSA_LIB_PATH=lib, LD_PRELOAD=sanitize.runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, f"ABI host checks failed under the sanitizers:\n{tail}"
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
