"""The C-ABI host code (argument checks, workspace layout and stash
planning, size queries) under AddressSanitizer and UndefinedBehaviorSanitizer:
the library is rebuilt with both sanitizers on the host side only (device
code unchanged), and the ABI tests run against it in a child process with
the ASan runtime preloaded.  Any report aborts that process, so the test
fails."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

from context_gqa_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_under_host_sanitizers(tmp_path):
    try:
        runtime = B.asan_runtime()
        B.hipcc()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = B.build_sanitized(str(tmp_path / "libdocmask_gqa_sanitized.so"))
    nm = shutil.which("nm")
    if nm:
        syms = subprocess.run([nm, "-D", lib], capture_output=True, text=True).stdout
        assert "__asan_" in syms and "__ubsan_" in syms, "the build is not instrumented"
    env = dict(os.environ, LD_PRELOAD=runtime, DMGQA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert " passed" in r.stdout and "failed" not in r.stdout
