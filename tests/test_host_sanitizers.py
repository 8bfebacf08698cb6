"""The host code of the library (C ABI validation and the zigzag plan) built
with AddressSanitizer and UndefinedBehaviorSanitizer, kernels stubbed out,
running the CPU tests of the ABI and the plan."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "branch_aware_causal_amd", "csrc")


@pytest.mark.slow
def test_abi_and_plan_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    lib = str(tmp_path / "libbac_sanitized.so")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", os.path.join(CSRC, "abi.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"), "-o", lib]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=asan, BAC_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          "-m", "not gpu", os.path.join(ROOT, "tests", "test_abi.py"),
                          os.path.join(ROOT, "tests", "test_accounting.py")],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    tail = (run.stdout + run.stderr)[-3000:]
    assert run.returncode == 0, tail
    assert "passed" in run.stdout and "AddressSanitizer" not in run.stderr, tail
