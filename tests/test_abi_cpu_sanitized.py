"""The host-side C-ABI checks of test_abi_cpu.py run again against a build of
the library whose host layer (argument validation, workspace sizing, launch
planning) is compiled with AddressSanitizer and UndefinedBehaviorSanitizer."""
import os
import subprocess
import sys

import pytest

from semi_autoregressive_drafting_amd import build as B
from semi_autoregressive_drafting_amd import dspark as D

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(B.asan_runtime() is None or not os.path.exists(D.LIB_PATH),
                    reason="needs the ROCm clang ASan runtime and a built libdspark.so")
def test_abi_checks_under_host_sanitizers():
    lib = B.build_host_sanitized()
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms  # the host layer is instrumented
    env = dict(os.environ, LD_PRELOAD=B.asan_runtime(), DSPARK_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                         env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    assert " passed" in res.stdout and "failed" not in res.stdout
