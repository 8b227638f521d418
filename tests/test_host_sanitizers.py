"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

A second copy of librtp is built with ASan + UBSan on its host pass only (device code
as usual), and the CPU tests of the C ABI (exports, descriptor and argument checks,
workspace sizing, the injected device failure) run against it in a child process with
the ASan runtime preloaded.  Any out-of-bounds access, use after free or undefined
behaviour in those host paths aborts the child with a report.
"""
import os
import subprocess
import sys

import pytest

from head_wise_sparse_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_code_under_asan_and_ubsan(tmp_path):
    try:
        lib = B.build_host_sanitized(str(tmp_path))
        runtime = B.asan_runtime()
    except RuntimeError as e:            # no HIP toolchain on this host
        pytest.skip(str(e))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the copy is not instrumented"
    env = dict(os.environ, LD_PRELOAD=runtime, RTP_LIB_PATH=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, f"CPU ABI tests under ASan/UBSan failed:\n{tail}"
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
