"""The host side of the C-ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

mla_verify_api.cpp (plan arithmetic, workspace layout, argument checks, the
launch sequence) is compiled with g++ for the host only, with the kernel
launches and the two HIP device queries stubbed (tests/host/sanitize_driver.cpp),
and driven through valid and invalid calls of every entry point.  Any
sanitizer report fails the run.  No GPU and no HIP runtime are involved.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_decoding_mla_page_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


def test_host_api_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if not gxx or not os.path.exists(os.path.join(ROCM_INCLUDE, "hip", "hip_runtime.h")):
        pytest.skip("g++ or the HIP headers are not available")
    exe = tmp_path / "sanitize_driver"
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", ROCM_INCLUDE]
    srcs = [os.path.join(CSRC, "mla_verify_api.cpp"), os.path.join(ROOT, "tests", "host", "sanitize_driver.cpp")]
    build = subprocess.run([gxx, *flags, *srcs, "-o", str(exe)], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0 and run.stdout.strip() == "ok", (run.stdout + run.stderr)[-3000:]
