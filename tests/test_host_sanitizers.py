"""Host C++ under the address and undefined-behaviour sanitizers (CPU only).

The staging planner (csrc/host_plan.cpp, plain C++ with no device code) is
compiled with g++ -fsanitize=address,undefined together with a randomised
driver (tests/host/plan_fuzz.cpp) that checks every plan's properties,
including the inputs a caller may get wrong (an expert in two slots, ids out
of range, more wanted experts than slots, null pointers). Any sanitizer
report aborts the driver.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "plan_fuzz")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "sparse_moe_decode_prerouter_amd", "csrc", "host_plan.cpp"),
           os.path.join(ROOT, "tests", "host", "plan_fuzz.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "plan_fuzz ok" in r.stdout
