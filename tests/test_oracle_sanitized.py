"""The oracle's pins re-run against an AddressSanitizer + UndefinedBehavior-
Sanitizer build of oracle/gdr_oracle.c (CPU only).  Any out-of-bounds
access, use of freed memory or undefined behaviour in the oracle aborts the
child run."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_oracle_pins_under_asan_and_ubsan():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    oracle.build(force=True, sanitized=True)
    env = dict(os.environ, GDR_ORACLE_SANITIZED="1", LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="4")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    log = res.stdout + res.stderr
    assert "AddressSanitizer" not in log and "runtime error" not in log, log[-4000:]
    assert res.returncode == 0, log[-4000:]
    assert " passed" in res.stdout
