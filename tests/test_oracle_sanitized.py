"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer:
the pins of the oracle (tests/test_oracle*.py) run again in a child process
that loads a sanitizer build of rosa_oracle.c.  Any out-of-bounds access,
use after free or undefined behaviour on those inputs aborts the child and
fails this test.  CPU only."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime():
    try:
        p = subprocess.run(["gcc", "-print-file-name=libasan.so"],
                           capture_output=True, text=True, timeout=30).stdout.strip()
    except (OSError, subprocess.SubprocessError):
        return None
    return p if p and os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_sanitizers():
    asan = _runtime()
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = oracle.build_sanitized()
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan, ROSA_ORACLE_LIB=lib,
               # the interpreter's own allocations are not the oracle's
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    tests = [os.path.join(ROOT, "tests", n) for n in
             ("test_oracle.py", "test_oracle_qk.py", "test_oracle_scatter.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x",
                        "-p", "no:cacheprovider", "-m", "not gpu", *tests],
                       cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=1200)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    for marker in ("AddressSanitizer", "runtime error:"):
        assert marker not in out, out[-4000:]
    assert " passed" in out
