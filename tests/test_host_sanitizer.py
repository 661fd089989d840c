"""The C entry points' host-side checks built with the address and
undefined-behaviour sanitizers (CPU only).

tests/host_asan/abi_checks.cpp calls every entry point of
csrc/flash_attn_api.cpp with bad and good arguments; the kernel launchers
are replaced by the stand-ins of tests/host_asan/launch_stub.cpp, so no GPU
code is built or run. Any sanitizer report aborts the program
(-fno-sanitize-recover), and a wrong status fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "io_aware_exact_11_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_asan")
ROCM_INCLUDE = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")


def test_entry_point_checks_under_asan_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM_INCLUDE, "hip", "hip_runtime.h")):
        pytest.skip("needs g++ and the HIP headers")
    exe = str(tmp_path / "abi_checks")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "flash_attn_api.cpp"), os.path.join(HERE, "launch_stub.cpp"),
           os.path.join(HERE, "abi_checks.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "all" in run.stdout and "checks passed" in run.stdout, out[-4000:]
