"""The host tests (C ABI argument checks, planners, oracle pins) run clean under
AddressSanitizer and UndefinedBehaviorSanitizer: tests/run_host_sanitizers.py builds
instrumented copies of the library's host code and of the oracle and runs them in a
child process, which any sanitizer report ends with a non-zero status."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(not glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"),
                    reason="clang sanitizer runtime not installed")
def test_host_code_clean_under_asan_and_ubsan():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "run_host_sanitizers.py"), "-x"],
                       cwd=ROOT, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, f"sanitizer run failed ({r.returncode}):\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    assert " passed" in r.stdout
