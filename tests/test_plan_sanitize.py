"""The library's host plan arithmetic (csrc/plan_host.cpp with the tile table and split
run arithmetic of csrc/tiles.hpp, which the kernels share) built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer and run through
tests/sanitize/plan_driver.cpp: argument rules, workspace layouts and the split-tail
schedule over a grid of problems. Any sanitizer report or failed check fails the test."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "gemm_epilogues_epilog_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_plan_arithmetic_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "plan_sanitized"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-Wall", "-Wextra",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "plan_host.cpp"), os.path.join(HERE, "sanitize", "plan_driver.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    for k in ("GE_TILE", "GE_STREAMK", "GE_PERSIST", "GE_SK_RUN", "GE_GROUP_M"):
        env.pop(k, None)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and "ok (0 failures)" in r.stdout, r.stdout[-3000:] + r.stderr[-4000:]
