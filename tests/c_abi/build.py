"""Builds skl_c_check, the plain-C driver of libstreamkl (host code only:
gcc, the HIP runtime and the library; no GPU needed to build)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "attention_kl_divergence_skl_amd")
SRC = os.path.join(HERE, "skl_c_check.c")
EXE = os.path.join(HERE, "skl_c_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_check() -> str:
    """Compiles and links skl_c_check against the in-tree libstreamkl.so
    (found at run time through an rpath relative to the executable)."""
    lib = os.path.join(PKG, "libstreamkl.so")
    if not os.path.exists(lib):
        raise RuntimeError("libstreamkl.so is not built")
    # The HIP runtime header needs its platform named when compiled by a C compiler.
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-L", PKG, "-lstreamkl", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../attention_kl_divergence_skl_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-o", EXE + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"building skl_c_check failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(EXE + ".tmp", EXE)
    return EXE
