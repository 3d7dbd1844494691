"""The C ABI's host code (validation, cutoff tables, host tile classifier,
tiling, compact-store geometry, dispatch) built with AddressSanitizer and
UndefinedBehaviorSanitizer and run on the CPU against host stand-ins of the
kernel launchers, which touch the first and last byte of every range each
launch would address (tests/host_check/).  A planted undersized buffer must
be reported, so the check is known to be live."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "host_check", "host_check")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(*args):
    if not os.path.exists(BIN):
        pytest.skip("sanitizer harness not built (python -m rope_positional_encoding_amd.build)")
    return subprocess.run([BIN, *args], capture_output=True, text=True, env=ENV, timeout=300)


def test_host_code_clean_under_sanitizers():
    r = _run()
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host_check ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_planted_overflow_is_reported():
    r = _run("undersized")
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr
