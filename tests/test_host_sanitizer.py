"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

libpsc_san.so is the host side of the library (argument checks, sizing,
workspace carving, status mapping) built with -fsanitize=address,undefined
and no device code.  The C-ABI tests of tests/test_abi.py, which need no GPU,
run in a subprocess against it (PSC_LIBRARY) with the ASan runtime preloaded;
any sanitizer report, or any failing test, fails this one.
"""
import os
import subprocess
import sys

import pytest

from packed_sequence_causal_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.slow


def test_abi_suite_under_host_sanitizers():
    if B.stale(B.LIB_SAN):
        B.build(release=False, sanitize=True)
    blob = open(B.LIB_SAN, "rb").read()
    assert b"__asan_init" in blob and b"__ubsan_handle" in blob, "libpsc_san.so is not instrumented"
    env = dict(os.environ)
    env.update(LD_PRELOAD=B.asan_runtime(), PSC_LIBRARY=B.LIB_SAN,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in r.stdout and " skipped" not in r.stdout, r.stdout[-2000:]
