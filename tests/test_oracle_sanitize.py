"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (g++, host
code only) and run through tests/sanitize/oracle_driver.cpp: every epilogue and storage
type, ragged m, transposed operands and several thread counts, each result also checked
against a direct float64 sum. Any sanitizer report aborts the driver and fails the test."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitized"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-pthread",
           os.path.join(ROOT, "oracle", "oracle.cpp"), os.path.join(HERE, "sanitize", "oracle_driver.cpp"),
           "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and "ok (0 failures)" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
