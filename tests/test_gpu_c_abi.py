"""The C ABI driven from plain C (tests/c_abi/skl_c_check.c): no Python
binding and no torch between the caller and libstreamkl.  The test writes a
seeded problem to a file, runs the program as a child process on the GPU, and
compares every output with the oracle; the joint call's gradients must also
equal the split calls' to the joint/split agreement bound."""
import os
import subprocess

import numpy as np
import pytest

from attention_kl_divergence_skl_amd import synth
from tests.c_abi.build import EXE, SRC, build_check
from tests.gpu_util import check_grad, check_rows, oracle_backward, oracle_forward, say

pytestmark = pytest.mark.gpu

CASES = [
    synth.Workload("c_f32_causal_d128_d64", 2, 2, 200, 333, 128, 64, "f32", True, 1 / np.sqrt(128), 1 / np.sqrt(64),
                   synth.Recipe("iid", amp1=2.0), "random", 31),
    synth.Workload("c_bf16_noncausal_d64_d128", 1, 3, 257, 190, 64, 128, "bf16", False, 1 / np.sqrt(64),
                   1 / np.sqrt(128), synth.Recipe("iid"), "random", 32),
    synth.Workload("c_bf16_causal_aligned", 1, 2, 256, 256, 128, 128, "bf16", True, 1 / np.sqrt(128),
                   1 / np.sqrt(128), synth.Recipe("corr", noise=0.3), "random", 33),
]


def _encode(a, dtype):
    """float32 values (bf16-representable for bf16 problems) as file bytes."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return a.tobytes()
    bits = a.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "bf16 inputs are exact in bf16"
    return (bits >> 16).astype(np.uint16).tobytes()


def _decode(buf, off, shape, dtype):
    n = int(np.prod(shape))
    if dtype == "f32":
        a = np.frombuffer(buf, np.float32, n, off)
        return a.reshape(shape), off + 4 * n
    u = np.frombuffer(buf, np.uint16, n, off).astype(np.uint32) << 16
    return u.view(np.float32).reshape(shape), off + 2 * n


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_plain_c_caller_matches_oracle(w, tmp_path):
    if not os.path.exists(EXE) or os.path.getmtime(EXE) < os.path.getmtime(SRC):
        build_check()
    say(f"[C ABI] {w.name}")
    x = synth.all_inputs(w)
    hdr = np.array([w.B, w.H, w.NQ, w.NK, w.d1, w.d2, int(w.causal), 0 if w.dtype == "bf16" else 1], np.int64)
    src = tmp_path / "in.bin"
    with open(src, "wb") as f:
        f.write(hdr.tobytes() + np.array([w.scale1, w.scale2], np.float32).tobytes())
        for k in ("q1", "k1", "q2", "k2"):
            f.write(_encode(x[k], w.dtype))
        f.write(np.ascontiguousarray(x["g"], np.float32).tobytes())
    dst = tmp_path / "out.bin"
    r = subprocess.run([EXE, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"skl_c_check failed ({r.returncode}): {r.stdout}{r.stderr}"
    buf = dst.read_bytes()
    rows = (w.B, w.H, w.NQ)
    off, got = 0, {}
    for k in ("kl", "lse1", "lse2"):
        got[k], off = _decode(buf, off, rows, "f32")
    shape = {"q1": (w.B, w.H, w.NQ, w.d1), "k1": (w.B, w.H, w.NK, w.d1),
             "q2": (w.B, w.H, w.NQ, w.d2), "k2": (w.B, w.H, w.NK, w.d2)}
    grads = []
    for name in ("q2", "k2", "q1", "k1", "q1", "k1", "q2", "k2"):
        g, off = _decode(buf, off, shape[name], w.dtype)
        grads.append(g.astype(np.float64))
    assert off == len(buf), "output size"
    check_rows(f"{w.name} (C)", w, got, oracle_forward(w, x))
    split = {"student": grads[0:2], "teacher": grads[2:4]}
    joint = {"teacher": grads[4:6], "student": grads[6:8]}
    for setting in ("student", "teacher"):
        rq, rk = oracle_backward(w, x, setting)
        for call, (dq, dk) in (("split", split[setting]), ("joint", joint[setting])):
            check_grad(f"{w.name} (C, {call}) dQ {setting}", w, dq, rq)
            check_grad(f"{w.name} (C, {call}) dK {setting}", w, dk, rk)
        rel = 1e-5 if w.dtype == "f32" else 2e-3
        for a, b in zip(split[setting], joint[setting]):
            # the two algorithms round dS differently (bf16 operands: 2^-9)
            assert np.linalg.norm(a - b) <= rel * np.linalg.norm(b) + 1e-6, f"{w.name}: joint vs split ({setting})"
