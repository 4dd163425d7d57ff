"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

gla_abi.cpp (validation, launch planning, scratch and timing bookkeeping) is
compiled with g++ -fsanitize=address,undefined together with
tests/abi_sanitize_driver.cpp, which stubs the kernel-launch layer and calls
every entry point on every validation error path (plus, when no GPU is
visible, a valid call that must return GLA_ERR_HIP).  Host code only: no GPU
code is built with a sanitizer.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("g++ or the HIP headers are missing")
    exe = str(tmp_path / "abi_sanitize")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "abi_sanitize_driver.cpp"),
           os.path.join(ROOT, "gated_bidirectional_linear_amd", "csrc", "gla_abi.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lamdhip64",
           "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    env = dict(os.environ)
    # the HIP runtime keeps allocations until exit: leak reports would be its own
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    print(run.stdout[-2000:])
    assert run.returncode == 0, run.stdout[-4000:] + run.stderr[-4000:]
    assert "ok (0 failures)" in run.stdout
