"""The C-ABI host code (api.cpp) under AddressSanitizer and
UndefinedBehaviorSanitizer: g++ builds it with stand-ins for the kernel
launchers and the HIP runtime calls (tests/sanitize/host_stubs.cpp) and a
harness that walks every entry point's validation, workspace sizing and
dispatch (tests/sanitize/host_abi_check.cpp).  Host code only; no GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "attention_kl_divergence_skl_amd", "csrc", "api.cpp"),
       os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp"),
       os.path.join(ROOT, "tests", "sanitize", "host_abi_check.cpp")]


def test_host_abi_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "host_abi_check")
    cmd = [gxx, "-std=c++17", "-g", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           *SRC, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "host ABI checks passed" in run.stdout
