"""The C-ABI layer (gqa_decode_api.cpp) built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer, host code only: the kernel
side is replaced by tests/c_abi/kernels_stub.cpp, and
tests/c_abi/sanitize_driver.cpp calls every entry point with the argument
errors the library must report (and a valid call, which reports the missing
device). No GPU is needed or used.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_abi_layer_is_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "sanitize_driver")
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "gqa_token_decode_amd", "csrc"),
           os.path.join(ROOT, "tests", "c_abi", "sanitize_driver.cpp"),
           os.path.join(ROOT, "tests", "c_abi", "kernels_stub.cpp"),
           os.path.join(ROOT, "gqa_token_decode_amd", "csrc", "gqa_decode_api.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr[-3000:]
    assert "0 mismatches" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr
