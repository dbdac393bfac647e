"""The autograd wrapper (attention_kl) over the C ABI: gradients of a weighted
sum of per-row KL with respect to all four inputs against the oracle, and a
frozen teacher (only Q2, K2 require gradients)."""
import numpy as np
import pytest
import torch

import oracle
from attention_kl_divergence_skl_amd import synth
from tests.gpu_util import check_grad, check_rows, say, to_device

pytestmark = pytest.mark.gpu


def W(name, B, H, NQ, NK, d1, d2, dtype, causal, recipe=synth.Recipe("corr", noise=0.4)):
    return synth.Workload(name, B, H, NQ, NK, d1, d2, dtype, causal, 1 / np.sqrt(d1), 1 / np.sqrt(d2),
                          recipe, "random", 3)


@pytest.mark.parametrize("algo", ["auto", "split", "joint"])
@pytest.mark.parametrize("w", [W("ag_bf16_causal", 1, 2, 300, 300, 128, 128, "bf16", True),
                               W("ag_f32_noncausal", 2, 1, 130, 200, 64, 128, "f32", False, synth.Recipe("iid"))],
                         ids=lambda w: w.name)
def test_autograd_gradients_of_all_inputs(gpu_lib, w, algo):
    say(f"[autograd {algo}] {w.name}")
    x, t = to_device(w)
    leaves = {k: t[k].clone().requires_grad_(True) for k in ("q1", "k1", "q2", "k2")}
    kl, lse1, lse2 = gpu_lib.attention_kl(leaves["q1"], leaves["k1"], leaves["q2"], leaves["k2"],
                                          w.scale1, w.scale2, w.causal, algo=algo)
    assert not lse1.requires_grad and not lse2.requires_grad
    (kl * t["g"]).sum().backward()
    torch.cuda.synchronize()
    ref = oracle.forward(x["q1"], x["k1"], x["q2"], x["k2"], w.scale1, w.scale2, w.causal)
    check_rows(w.name, w, {"kl": kl.detach().cpu().numpy(), "lse1": lse1.cpu().numpy(),
                           "lse2": lse2.cpu().numpy()}, ref)
    dq2, dk2 = oracle.backward(x["q1"], x["k1"], x["q2"], x["k2"], w.scale1, w.scale2, w.causal, x["g"],
                               "student")
    dq1, dk1 = oracle.backward(x["q1"], x["k1"], x["q2"], x["k2"], w.scale1, w.scale2, w.causal, x["g"],
                               "teacher")
    for name, ref_g in (("q1", dq1), ("k1", dk1), ("q2", dq2), ("k2", dk2)):
        g = leaves[name].grad
        assert g is not None and g.dtype == leaves[name].dtype and g.shape == leaves[name].shape
        check_grad(f"{w.name} d{name}", w, g.float().cpu().numpy(), ref_g)


def test_autograd_frozen_teacher(gpu_lib):
    w = W("ag_frozen_teacher", 1, 2, 200, 200, 128, 64, "bf16", True, synth.Recipe("iid", amp1=2.0))
    say(f"[autograd] {w.name}")
    x, t = to_device(w)
    q2 = t["q2"].clone().requires_grad_(True)
    k2 = t["k2"].clone().requires_grad_(True)
    kl, _, _ = gpu_lib.attention_kl(t["q1"], t["k1"], q2, k2, w.scale1, w.scale2, True)
    kl.mean().backward()
    torch.cuda.synchronize()
    g = np.full((w.B, w.H, w.NQ), 1.0 / (w.B * w.H * w.NQ))
    rq, rk = oracle.backward(x["q1"], x["k1"], x["q2"], x["k2"], w.scale1, w.scale2, True, g, "student")
    check_grad("frozen teacher dq2", w, q2.grad.float().cpu().numpy(), rq)
    check_grad("frozen teacher dk2", w, k2.grad.float().cpu().numpy(), rk)


def test_autograd_key_broadcast_over_heads(gpu_lib):
    """K1 shared by all heads through expand() (a stride of 0 on the head
    axis): its gradient is the sum over heads of the per-head dK1.  The C ABI
    itself rejects such a layout for the gradient it would write in place."""
    w = W("ag_broadcast_k1", 2, 3, 200, 260, 64, 64, "bf16", True, synth.Recipe("iid", amp1=2.0))
    say(f"[autograd] {w.name}")
    x, t = to_device(w)
    k1_shared = x["k1"][:, :1]                                     # [B, 1, NK, d1]
    k1_full = np.ascontiguousarray(np.broadcast_to(k1_shared, x["k1"].shape))
    base = torch.from_numpy(np.ascontiguousarray(k1_shared)).to(torch.bfloat16).cuda().requires_grad_(True)
    k1 = base.expand(w.B, w.H, w.NK, w.d1)
    assert k1.stride(1) == 0
    q2 = t["q2"].clone().requires_grad_(True)
    kl, _, _ = gpu_lib.attention_kl(t["q1"], k1, q2, t["k2"], w.scale1, w.scale2, True)
    (kl * t["g"]).sum().backward()
    torch.cuda.synchronize()
    _, dk1 = oracle.backward(x["q1"], k1_full, x["q2"], x["k2"], w.scale1, w.scale2, True, x["g"], "teacher")
    dq2, _ = oracle.backward(x["q1"], k1_full, x["q2"], x["k2"], w.scale1, w.scale2, True, x["g"], "student")
    check_grad("broadcast k1 grad", w, base.grad.float().cpu().numpy(), dk1.sum(axis=1, keepdims=True))
    check_grad("broadcast k1: dq2", w, q2.grad.float().cpu().numpy(), dq2)
    kl2, l1, l2 = gpu_lib.skl_forward(t["q1"], k1.detach(), t["q2"], t["k2"], w.scale1, w.scale2, True)
    with pytest.raises(gpu_lib.SklError) as e:
        gpu_lib.skl_backward_teacher(t["q1"], k1.detach(), t["q2"], t["k2"], l1, l2, kl2, t["g"],
                                     w.scale1, w.scale2, True)
    assert e.value.status == 2


def test_autograd_without_query_rows(gpu_lib):
    """An empty query block: KL has no rows and every input gradient is
    zero (the key gradients have rows and are written as zeros)."""
    say("[autograd] no query rows")
    g = torch.Generator(device="cpu").manual_seed(9)
    k1 = torch.randn(1, 2, 40, 64, generator=g).to("cuda", torch.bfloat16).requires_grad_()
    k2 = torch.randn(1, 2, 40, 64, generator=g).to("cuda", torch.bfloat16).requires_grad_()
    q1 = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device="cuda", requires_grad=True)
    q2 = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device="cuda", requires_grad=True)
    kl, _, _ = gpu_lib.attention_kl(q1, k1, q2, k2, causal=True)
    assert kl.shape == (1, 2, 0)
    kl.sum().backward()
    for t in (q1, k1, q2, k2):
        assert t.grad is not None and t.grad.shape == t.shape
        assert torch.equal(t.grad, torch.zeros_like(t.grad))
