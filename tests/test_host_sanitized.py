"""The planner's host code built with g++ -fsanitize=address,undefined and
driven through its whole configuration space (tests/host/plan_selftest.cpp):
error paths, grid coverage, scratch bounds and bucket invariants.  CPU only."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_plan_selftest_under_asan_ubsan(tmp_path):
    exe = tmp_path / "plan_selftest"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "host", "plan_selftest.cpp"),
           os.path.join(ROOT, "fp8_paged_kv_pa_amd", "csrc", "plan.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300,
                       env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
    assert r.returncode == 0, r.stdout + r.stderr
    assert "plan self-test ok" in r.stdout
