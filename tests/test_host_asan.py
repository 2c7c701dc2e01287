"""The library's host-only code under AddressSanitizer and UndefinedBehaviorSanitizer.

The host source (argument checks, path decision, pipeline schedule, threshold search, tuning
tables and files) is compiled with g++ together with tests/asan/host_driver.cpp, which calls
every host-only entry point on valid and invalid inputs; any sanitizer report fails the test.
GPU code is not built here (the sanitizers apply to host code only).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_SRC = os.path.join(ROOT, "projection_residual_rmsnorm_amd", "csrc", "pr_host.cpp")
DRIVER = os.path.join(ROOT, "tests", "asan", "host_driver.cpp")


def test_host_code_is_sanitizer_clean(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "host_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           HOST_SRC, DRIVER, "-o", exe]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0 and "asan" in proc.stderr.lower():
        pytest.skip("the sanitizer runtime is not installed: " + proc.stderr[-300:])
    assert proc.returncode == 0, proc.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe, str(tmp_path / "tuning.txt")], capture_output=True, text=True,
                         env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "AddressSanitizer" not in run.stderr and "runtime error" not in run.stderr, run.stderr
    assert "calls succeeded" in run.stdout
