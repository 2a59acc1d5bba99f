"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with the host side instrumented (device code as
usual) and the CPU C-ABI tests (symbol exports, host helpers, every argument
check and its error status) run against it in a child process with the clang
ASan runtime preloaded.  Any heap overflow, use after free or undefined
behaviour in the argument checks, workspace layouts or chunk rules stops the
child with a sanitizer report.
"""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

from token_block_sparsification_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_abi_cpu_tests_clean_under_host_sanitizers():
    tmp = tempfile.mkdtemp(prefix="up_asan_")
    lib = B.build(out=os.path.join(tmp, "libuniprefill_asan.so"), objdir=tmp, host_sanitize=True)
    env = dict(os.environ)
    env.update(UNIPREFILL_LIBRARY=lib, LD_PRELOAD=B.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    try:
        p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                           cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                           text=True, timeout=900)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    out = p.stdout
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert p.returncode == 0, out[-4000:]
    assert " passed" in out
