"""Build libstreamkl.so in-tree with hipcc for gfx950.

    python -m attention_kl_divergence_skl_amd.build [-j N]

Each translation unit is compiled to an object in parallel, then linked into
``attention_kl_divergence_skl_amd/libstreamkl.so``.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libstreamkl.so")
SOURCES = ["api.cpp", "fwd.hip", "bwd.hip", "bwd_split.hip", "bwd_joint.hip", "noalloc.hip"]
ARCH = "gfx950"

# Packed fp32 ops (v_pk_fma_f32 & co.) are switched off for all device code.
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    "-I", os.path.join(ROOT, "include"),
]

# Per-source additions.  The forward's running max is an fmaxf tree over MFMA
# results; under IEEE NaN semantics every operand is first quieted with an
# extra v_max_f32 (one VALU op per logit, about a sixth of the kernel's VALU
# work).  The forward never produces a NaN that it consumes: masked logits are
# -inf and are selected away before any inf - inf is used, and the running
# maxima start at the finite kNoKey = -1e30 (so a lane whose keys are all
# masked keeps finite shifts); it is therefore compiled without NaN semantics.
SOURCE_FLAGS = {"fwd.hip": ["-fno-honor-nans"]}


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [_hipcc()] + HIPCC_FLAGS + SOURCE_FLAGS.get(src, []) + list(extra) + lang
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    noise = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(jobs: int = 8, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", "--jobs", type=int, default=min(8, os.cpu_count() or 1))
    args = ap.parse_args(argv)
    print(build(args.jobs))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
