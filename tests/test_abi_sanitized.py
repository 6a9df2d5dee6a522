"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the library is rebuilt with its host code instrumented, and every
ctypes-level case of test_abi.py (symbols, workspace sizes, each invalid
argument of each entry point, enum values outside the enumerators) runs
against it in a child process with the sanitizer runtime preloaded. Any
sanitizer report fails the child (UBSan does not recover; ASan halts)."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_cases_clean_under_host_sanitizers():
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    sys.path.insert(0, ROOT)
    from linear_attention_05_amd import build
    lib = build.build_host_sanitized()
    env = dict(os.environ, LD_PRELOAD=build.sanitizer_runtime(), KDA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # the two cases that go through torch tensors test Python checks only
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
           "-p", "no:cacheprovider", "-k", "not binding_refuses and not binding_rejects"]
    res = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "Sanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
