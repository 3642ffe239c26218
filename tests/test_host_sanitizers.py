"""The C ABI layer's host code (load-time scale check, argument checks,
workspace sizing, launch sequencing) built with g++ under AddressSanitizer
and UndefinedBehaviorSanitizer against recording stubs of the kernels and of
the two HIP runtime calls it makes, then run: tests/host/abi_host_checks.cpp.
CPU only; no GPU and no HIP runtime involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIP_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or
                    not os.path.exists(os.path.join(HIP_INCLUDE, "hip", "hip_runtime.h")),
                    reason="needs g++ and the HIP headers")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_host_checks")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I" + HIP_INCLUDE, "-I" + ROOT,
           os.path.join(ROOT, "nvfp4_w4a4_expert_amd", "csrc", "api.cpp"),
           os.path.join(ROOT, "tests", "host", "abi_host_checks.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "abi host checks ok" in r.stdout
