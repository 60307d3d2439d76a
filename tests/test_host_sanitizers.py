"""The library's host-side model description (configuration validation and
defaults, parameter table, learning-rate schedule: csrc/host_model.cpp, the
same source libgpt.so compiles) built alone with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer, with a driver that checks the parameter counts the
Lecture prints, the table's layout invariants, the rejected configurations,
a fuzz of configurations and the schedule (CPU only; no GPU code involved)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_model_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = tmp_path / "host_model_check"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "transformer_lm_step_gpt_amd", "csrc", "host_model.cpp"),
           os.path.join(ROOT, "tests", "host", "host_model_check.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert r.stdout.strip().splitlines()[-1] == "ok", r.stdout[-4000:]
