"""The C ABI's host code (argument validation, workspace carving, status
mapping) built for the CPU with g++ under the address and undefined-
behaviour sanitizers, against a stand-in for the kernel launch layer that
records each launch (tests/hostcheck). No GPU and no HIP runtime call is
involved: api.cpp calls HIP only through the launch layer."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HC = os.path.join(ROOT, "tests", "hostcheck")
ROCM_INC = "/opt/rocm/include"


def test_abi_host_code_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(ROCM_INC):
        pytest.skip("g++ or the ROCm headers are missing")
    exe = str(tmp_path / "host_check")
    # host-only build: g++ compiles api.cpp and the stand-in; no device code
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    cmd = [gxx, "-std=c++17", "-O1", "-g", *san, "-Wall", "-Wextra", "-Wno-unused-parameter",
           "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INC, "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "mxfp4_quantized_gemm_amd", "csrc", "api.cpp"),
           os.path.join(HC, "launch_stub.cpp"), os.path.join(HC, "host_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "checks passed" in r.stdout
