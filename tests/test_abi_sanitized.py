"""The C-ABI's argument validation built for the host with AddressSanitizer
and UndefinedBehaviorSanitizer (g++, no device code: the kernel launchers
are stubs that fail if reached), driven through every rejected-argument
case.  Needs no GPU."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "entropic_ot_banded_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "abi_sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.timeout(300)
def test_validation_layer_under_asan_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("g++ or the HIP headers are missing")
    exe = str(tmp_path / "abi_sanitized")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "api.cpp"), os.path.join(HERE, "stubs.cpp"), os.path.join(HERE, "driver.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lamdhip64", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=240)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "all checks passed" in run.stdout
