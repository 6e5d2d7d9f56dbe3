"""The oracle's pin and cross-check suites run again against a build of the
same C source with AddressSanitizer and UndefinedBehaviorSanitizer, any
finding aborting the run: an out-of-bounds read, a use after free or an
integer overflow in the oracle would otherwise go unseen by tests that only
compare values.  The suites run in a child process with the sanitizer
runtime preloaded (the Python interpreter itself is not instrumented)."""
import os
import shutil
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime():
    gcc = shutil.which("gcc")
    if not gcc:
        return None
    path = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_suites_pass_under_address_and_ub_sanitizers(tmp_path):
    asan = _runtime()
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    env = dict(os.environ, ALHR_ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py", "tests/test_oracle_transcription.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = "\n".join((r.stdout + r.stderr).splitlines()[-30:])
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "failed" not in r.stdout, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
