"""The host schedulers under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/native/schedule_fuzz.cpp drives pkvmla_schedule.cpp (pure C++, no GPU
code) through random flat, two-level and one-launch cascade cases and checks
coverage and slot invariants; it is compiled with g++ and both sanitizers on
the CPU (the GPU kernels are not part of this build)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_mla_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_schedulers_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "schedule_fuzz"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", f"-I{CSRC}",
           os.path.join(ROOT, "tests", "native", "schedule_fuzz.cpp"),
           os.path.join(CSRC, "pkvmla_schedule.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe), "1500"], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
