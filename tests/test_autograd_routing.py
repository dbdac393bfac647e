"""CPU tests of attention_kl's routing (no GPU): which backward calls the
autograd wrapper makes for which inputs needing gradients, with the library
calls replaced by recording stand-ins that return zeros of the right shapes."""
import pytest
import torch

import attention_kl_divergence_skl_amd as skl


@pytest.fixture
def calls(monkeypatch):
    log = []

    def forward(q1, k1, q2, k2, s1, s2, causal):
        B, H, N = q1.shape[:3]
        z = torch.zeros(B, H, N)
        return z + 0.25, z.clone(), z.clone()

    def student(q1, k1, q2, k2, l1, l2, g, s1, s2, causal, algo="split", ws=None):
        log.append(("student", algo))
        return torch.zeros_like(q2), torch.zeros_like(k2)

    def teacher(q1, k1, q2, k2, l1, l2, kl, g, s1, s2, causal, algo="split", ws=None):
        log.append(("teacher", algo))
        return torch.zeros_like(q1), torch.zeros_like(k1)

    def joint(q1, k1, q2, k2, l1, l2, kl, g, s1, s2, causal, ws=None):
        log.append(("joint",))
        return tuple(torch.zeros_like(x) for x in (q1, k1, q2, k2))

    monkeypatch.setattr(skl, "skl_forward", forward)
    monkeypatch.setattr(skl, "skl_backward_student", student)
    monkeypatch.setattr(skl, "skl_backward_teacher", teacher)
    monkeypatch.setattr(skl, "skl_backward_joint", joint)
    return log


def _inputs(grad_teacher=True, grad_student=True):
    t = [torch.randn(1, 2, 5, 8) for _ in range(4)]
    for i, x in enumerate(t):
        x.requires_grad_(grad_teacher if i < 2 else grad_student)
    return t


def _run(algo, **kw):
    q1, k1, q2, k2 = _inputs(**kw)
    kl, _, _ = skl.attention_kl(q1, k1, q2, k2, causal=True, algo=algo)
    kl.sum().backward()
    return q1, k1, q2, k2


@pytest.mark.parametrize("algo", ["auto", "joint"])
def test_both_settings_make_one_joint_call(calls, algo):
    q1, k1, q2, k2 = _run(algo)
    assert calls == [("joint",)]
    assert all(x.grad is not None and x.grad.shape == x.shape for x in (q1, k1, q2, k2))


def test_split_forces_the_two_calls(calls):
    _run("split")
    assert calls == [("student", "split"), ("teacher", "split")]


@pytest.mark.parametrize("algo", ["auto", "joint"])
def test_one_setting_makes_one_split_call(calls, algo):
    q1, k1, q2, k2 = _run(algo, grad_teacher=False)  # frozen teacher
    assert calls == [("student", "split")]
    assert q1.grad is None and k1.grad is None and q2.grad is not None and k2.grad is not None
    calls.clear()
    _run(algo, grad_student=False)
    assert calls == [("teacher", "split")]


def test_fused_atomic_passes_through(calls):
    _run("fused_atomic")
    assert calls == [("student", "fused_atomic"), ("teacher", "fused_atomic")]


def test_unknown_algorithm_is_rejected_before_any_call(calls):
    q1, k1, q2, k2 = _inputs()
    with pytest.raises(skl.SklError):
        skl.attention_kl(q1, k1, q2, k2, algo="fastest")
    assert calls == []
