"""A fixed, seeded sweep of random small shapes through the forward, both
backward settings (student and teacher calls) and the joint backward call
against the oracle.  The kernels decide per step whether masking is needed
(causal diagonal, ragged query and key edges) and, with few query tiles,
split the dQ kernel's keys into ranges; random N_Q, N_K, head dims, recipes
and dtypes exercise those decisions together."""
import numpy as np
import pytest
import torch

from attention_kl_divergence_skl_amd import synth
from tests.gpu_util import check_grad, check_rows, gpu_forward, grad_to_np, oracle_backward, oracle_forward, say, to_device

pytestmark = pytest.mark.gpu


def _shapes(n=24, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        causal = bool(rng.integers(0, 2))
        nq = int(rng.integers(1, 700))
        nk = int(rng.integers(nq if causal else 1, 900))
        d1, d2 = (int(x) for x in rng.choice([64, 128], 2))
        dtype = "f32" if rng.random() < 0.25 else "bf16"
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        recipe = synth.Recipe("corr", noise=0.4) if d1 == d2 and rng.random() < 0.5 else \
            synth.Recipe("iid", amp1=float(rng.choice([1.0, 3.0])))
        out.append(synth.Workload(f"rand{i}_{'c' if causal else 'n'}_{nq}x{nk}_{d1}_{d2}_{dtype}", B, H, nq, nk,
                                  d1, d2, dtype, causal, 1 / np.sqrt(d1), 1 / np.sqrt(d2), recipe, "random",
                                  1000 + i))
    return out


@pytest.mark.parametrize("w", _shapes(), ids=lambda w: w.name)
def test_random_shape(gpu_lib, w):
    say(f"[random shape] {w.name} B{w.B} H{w.H}")
    x, t = to_device(w)
    got, (kl, l1, l2) = gpu_forward(gpu_lib, w, t)
    check_rows(w.name, w, got, oracle_forward(w, x))
    dq2, dk2 = gpu_lib.skl_backward_student(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, t["g"],
                                            w.scale1, w.scale2, w.causal)
    dq1, dk1 = gpu_lib.skl_backward_teacher(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, kl, t["g"],
                                            w.scale1, w.scale2, w.causal)
    none = torch.empty(0, dtype=torch.float32, device="cuda")  # no workspace: the joint kernels themselves
    jq1, jk1, jq2, jk2 = gpu_lib.skl_backward_joint(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, kl, t["g"],
                                                    w.scale1, w.scale2, w.causal, ws=none)
    torch.cuda.synchronize()
    for setting, dq, dk, jq, jk in (("student", dq2, dk2, jq2, jk2), ("teacher", dq1, dk1, jq1, jk1)):
        rq, rk = oracle_backward(w, x, setting)
        check_grad(f"{w.name} dQ ({setting})", w, grad_to_np(dq), rq)
        check_grad(f"{w.name} dK ({setting})", w, grad_to_np(dk), rk)
        check_grad(f"{w.name} joint dQ ({setting})", w, grad_to_np(jq), rq)
        check_grad(f"{w.name} joint dK ({setting})", w, grad_to_np(jk), rk)
