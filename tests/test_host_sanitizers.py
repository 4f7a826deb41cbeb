"""The C ABI's host code (argument checks, sizing, level offsets, launch planning: csrc/api.cpp)
built for the CPU with AddressSanitizer and UndefinedBehaviorSanitizer, its kernel launches
replaced by no-ops (tests/asan/host_stubs.cpp), and driven through many shapes and calls by
tests/asan/abi_host_check.cpp. No GPU is involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_hierarchical_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"),
                    reason="needs g++ and the HIP headers")
def test_abi_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_host_check")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           "-I" + CSRC, os.path.join(CSRC, "api.cpp"), os.path.join(ROOT, "tests", "asan", "host_stubs.cpp"),
           os.path.join(ROOT, "tests", "asan", "abi_host_check.cpp"), "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout[-2000:], r.stderr[-4000:])
