"""The library's host code (byte model, arena layout, planner, argument checks) built with g++
and AddressSanitizer into a small harness (asan_host_harness.cpp) and run on random shapes,
plans and budgets: no memory error, and every status as expected."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_kv_decode_amd", "csrc")
ROCM = "/opt/rocm"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")),
                    reason="needs g++ and the HIP runtime library to link against")
def test_host_code_under_address_sanitizer(tmp_path):
    exe = str(tmp_path / "harness")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-x", "c++", os.path.join(CSRC, "planner.cpp"), os.path.join(CSRC, "loopkv_api.cpp"),
           os.path.join(ROOT, "tests", "asan_host_harness.cpp"), "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "0 unexpected statuses" in r.stdout
