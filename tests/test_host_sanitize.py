"""The host planner and validator under AddressSanitizer and UBSan (CPU only):
a g++ build of the planner source with a fuzz driver, run over thousands of
random length sets, exact and undersized buffers and corrupted plans."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_planner_under_asan_ubsan(tmp_path):
    exe = tmp_path / "plan_fuzz"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "host", "plan_fuzz.cpp"),
           os.path.join(ROOT, "load_balanced_split_step_amd", "csrc", "hda_plan.cpp"),
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([str(exe), "20000"], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "clean" in r.stdout
