"""The host code of libcpattn (planners and the argument validation in front
of every launch) under AddressSanitizer and UndefinedBehaviorSanitizer.

plan.cpp and api.cpp are compiled with g++ together with a driver
(sanitize/host_checks.cpp) and stand-ins for the HIP runtime calls and the
kernel launchers (sanitize/launch_stubs.cpp), so no GPU is involved: the
driver runs the planners over random, edge and invalid inputs and every
device call with valid and invalid descriptors, checking statuses and that
rejected calls launch nothing. Any memory error or undefined behaviour
aborts the run."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "context_attention_long_amd", "csrc")
ROCM_INCLUDE = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")


def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("g++ or the ROCm headers are not available")
    exe = str(tmp_path / "host_checks")
    cmd = [gxx, "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I" + ROCM_INCLUDE, "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
           "-x", "c++", os.path.join(CSRC, "plan.cpp"), "-x", "c++", os.path.join(CSRC, "api.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "host checks passed" in run.stdout
