"""The oracle built with the address and undefined-behaviour sanitizers.

tests/sanitize/oracle_driver.c runs every step function of oracle/oracle.c on
small inputs that reach its edge cases. It is built twice with gcc, plain and
with -fsanitize=address,undefined (no recovery), and run in subprocesses: the
sanitized run must exit cleanly with no sanitizer report, and print exactly
what the plain build prints (a result that depends on undefined behaviour or
uninitialised memory would differ)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c")


def _build(tmp_path, name, flags):
    exe = str(tmp_path / name)
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
                           "-Wall", "-Wno-unknown-pragmas", *flags, SRC, DRIVER, "-o", exe, "-lm"])
    return exe


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    plain = _build(tmp_path, "plain", [])
    san = _build(tmp_path, "san", ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                                   "-fno-omit-frame-pointer"])
    # verify_asan_link_order=0: the environment may preload another library
    # ahead of the sanitizer runtime; the run is still fully instrumented
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    a = subprocess.run([plain], capture_output=True, text=True, timeout=120)
    b = subprocess.run([san], capture_output=True, text=True, timeout=300, env=env)
    assert a.returncode == 0, a.stdout + a.stderr
    assert b.returncode == 0, b.stderr[-4000:]
    assert "runtime error" not in b.stderr and "AddressSanitizer" not in b.stderr, b.stderr[-4000:]
    assert a.stdout == b.stdout
    assert a.stdout.count("rc=0") == 6 * 6
