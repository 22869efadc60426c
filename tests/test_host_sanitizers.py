"""The library's host (offline) code built with AddressSanitizer and
UndefinedBehaviorSanitizer (g++, no HIP) and driven over seeded random layers,
act order, per-channel groups, symmetric and 8-bit weights and refused arguments
(tests/native/host_sanitize.cpp).  Any sanitizer finding fails the test."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "w4a16_gemm_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ is not available")
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "host_sanitize"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "host.cpp"), os.path.join(ROOT, "tests", "native", "host_sanitize.cpp"),
           "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, (run.stdout + run.stderr)[-6000:]
    assert "0 failures" in run.stdout
