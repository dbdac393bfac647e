"""GPU parity at the full evaluation sizes, through the same entry points
bench.py times (the forward, the joint backward call it times by default, and
the student and teacher calls of its split mode).  The oracle checks sampled rows exactly (each row's KL, LSE
and dQ only need that row), sampled key columns near the end of causal
sequences (few rows see them), whole heads at 16K (every row and key column
of dQ and dK), the first key columns at 64K (every query row sees them, so the
dK kernel walks all query tiles for them), and, for every head, properties
that hold at any size: the key gradients of a head sum to zero, and
sum_i <q_i, dQ_i> equals sum_j <k_j, dK_j> (both are scale * sum dS (q . k))."""
import numpy as np
import pytest
import torch

import oracle
from attention_kl_divergence_skl_amd import synth
from tests.gpu_util import TOL, check_grad, check_rows_grad, rel_l2, say

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


def sample_rows(n, seed=0, k=24):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 127, 128, n // 2, n - 129, n - 128, n - 2, n - 1]
    return np.unique(np.concatenate([[r for r in fixed if 0 <= r < n], rng.integers(0, n, k)]))


@pytest.fixture(scope="module")
def store():
    return {}


def inputs(store, name):
    if name not in store:
        store.clear()
        torch.cuda.empty_cache()
        w = synth.WORKLOADS[name]
        say(f"[full] generating {name}")
        store[name] = (w, synth.device_inputs(w, "cuda"))
        torch.cuda.synchronize()
    return store[name]


def heads_to_check(w):
    return sorted({(0, 0), (w.B - 1, w.H - 1), (0, w.H // 2)})


def check_sampled_forward(w, kl, l1, l2, rows_seed=0):
    tol = TOL[w.dtype]
    for b, h in heads_to_check(w):
        q1, k1, q2, k2 = synth.head_inputs(w, b, h)
        rows = sample_rows(w.NQ, rows_seed + 7 * h)
        ref = oracle.head_forward(q1, k1, q2, k2, w.scale1, w.scale2, w.causal, rows)
        got = {k: v[b, h].cpu().numpy()[rows].astype(np.float64) for k, v in (("kl", kl), ("lse1", l1), ("lse2", l2))}
        err = np.abs(got["kl"] - ref["kl"])
        assert np.all(err <= tol["kl_abs"] + tol["kl_rel"] * np.abs(ref["kl"])), \
            f"{w.name} head ({b},{h}): KL err {err.max():.3e}"
        for k in ("lse1", "lse2"):
            assert np.abs(got[k] - ref[k]).max() <= tol["lse"], f"{w.name} ({b},{h}) {k}"


def check_dq_dk_identity(w, q, k, dq, dk, setting):
    """Property at any size, for every head: sum_i <q_i, dQ_i> and
    sum_j <k_j, dK_j> of the optimised side are both scale * sum_ij dS_ij
    (q_i . k_j), so they agree up to rounding (the two kernels recompute dS
    separately and round it to bf16 on their own).  A dK tile that is missing,
    wrongly scaled or given the wrong operand breaks the equality."""
    a = (q.double() * dq.double()).sum(dim=(2, 3))
    b = (k.double() * dk.double()).sum(dim=(2, 3))
    mag = (q.double() * dq.double()).abs().sum(dim=(2, 3)) + (k.double() * dk.double()).abs().sum(dim=(2, 3))
    err = ((a - b).abs() / mag).max().item()
    tag = f"{w.name}{'' if w.causal else ' without the mask'} ({setting})"
    say(f"[full] {tag}: sum <q, dQ> vs sum <k, dK>, worst head {err:.2e} of the term magnitude")
    # Measured about 2e-6 at 64K; a missing key tile moves it by percents and a
    # 1 % error in dK's scale by about 1e-3.
    assert err <= 1e-4, f"{tag}: dQ / dK identity off by {err:.3e}"


def check_sampled_backward(w, dq, dk, setting, early_cols_head=None, t=None):
    """Sampled dQ rows and trailing dK columns of a few heads; with
    early_cols_head = (b, h), also key columns 0..31 of that head, which every
    query row sees (the oracle materialises all rows for them); with the
    device inputs t, the dQ / dK identity for every head."""
    tol = TOL[w.dtype]["grad"]
    dq_np = dq.float()
    dk_np = dk.float()
    for b, h in heads_to_check(w):
        q1, k1, q2, k2 = synth.head_inputs(w, b, h)
        g = synth.head_grad(w, b, h)
        rows = sample_rows(w.NQ, 11 + h)
        rq = oracle.head_dq_rows(q1, k1, q2, k2, w.scale1, w.scale2, w.causal, g, setting, rows)
        got = dq_np[b, h].cpu().numpy()[rows]
        e = rel_l2(got, rq)
        assert e <= tol, f"{w.name} ({b},{h}) sampled dQ ({setting}) rel L2 {e:.3e}"
        check_rows_grad(f"{w.name} ({b},{h}) sampled dQ ({setting})", tol, got, rq)
        if w.causal:
            cols = np.arange(w.NK - 48, w.NK)
            rk = oracle.head_dk_cols(q1, k1, q2, k2, w.scale1, w.scale2, w.causal, g, setting, cols)
            got = dk_np[b, h].cpu().numpy()[cols]
            e = rel_l2(got, rk)
            assert e <= tol, f"{w.name} ({b},{h}) sampled dK ({setting}) rel L2 {e:.3e}"
            check_rows_grad(f"{w.name} ({b},{h}) trailing dK ({setting})", tol, got, rk)
    if early_cols_head is not None:
        b, h = early_cols_head
        say(f"[full] {w.name} ({b},{h}) dK key columns 0..31 ({setting}) against the oracle")
        q1, k1, q2, k2 = synth.head_inputs(w, b, h)
        g = synth.head_grad(w, b, h)
        cols = np.arange(32)
        rk = oracle.head_dk_cols(q1, k1, q2, k2, w.scale1, w.scale2, w.causal, g, setting, cols)
        got = dk_np[b, h].cpu().numpy()[cols]
        e = rel_l2(got, rk)
        assert e <= tol, f"{w.name} ({b},{h}) early dK ({setting}) rel L2 {e:.3e}"
        er = check_rows_grad(f"{w.name} ({b},{h}) early dK ({setting})", tol, got, rk)
        say(f"[full] early dK columns: rel L2 {e:.2e}, worst column {er:.2e}")
    if t is not None:
        side = "1" if setting == "teacher" else "2"
        check_dq_dk_identity(w, t["q" + side], t["k" + side], dq, dk, setting)
    # Property at any size: sum_j dK[j] = 0 for every head.
    s = dk.double().sum(dim=2).norm(dim=-1)
    f = dk.double().norm(dim=(2, 3))
    assert torch.all(s <= 1e-2 * f + 1e-30), f"{w.name}: key gradients do not sum to zero ({setting})"
    assert torch.isfinite(dq_np).all() and torch.isfinite(dk_np).all()


def backward_calls(gpu_lib, t, w, kl, l1, l2, causal):
    """(setting, dq, dk) for the student call, the teacher call and both
    settings of one joint call, one call at a time (each frees before the next)."""
    for call in ("student", "teacher", "joint"):
        say(f"[full] {w.name} {call} backward causal={causal}")
        if call == "student":
            dq, dk = gpu_lib.skl_backward_student(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, t["g"],
                                                  w.scale1, w.scale2, causal)
            torch.cuda.synchronize()
            yield "student", dq, dk
            del dq, dk
        elif call == "teacher":
            dq, dk = gpu_lib.skl_backward_teacher(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, kl, t["g"],
                                                  w.scale1, w.scale2, causal)
            torch.cuda.synchronize()
            yield "teacher", dq, dk
            del dq, dk
        else:
            dq1, dk1, dq2, dk2 = gpu_lib.skl_backward_joint(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, kl, t["g"],
                                                            w.scale1, w.scale2, causal)
            torch.cuda.synchronize()
            yield "teacher", dq1, dk1
            del dq1, dk1
            yield "student", dq2, dk2
            del dq2, dk2


def test_causal_4k_all_settings(gpu_lib, store):
    w, t = inputs(store, "causal_4k_h8x2_d128_corr03")
    say("[full] causal 4K forward + both backward settings")
    kl, l1, l2 = gpu_lib.skl_forward(t["q1"], t["k1"], t["q2"], t["k2"], w.scale1, w.scale2, w.causal)
    dq2, dk2 = gpu_lib.skl_backward_student(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, t["g"],
                                            w.scale1, w.scale2, w.causal)
    dq1, dk1 = gpu_lib.skl_backward_teacher(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, kl, t["g"],
                                            w.scale1, w.scale2, w.causal)
    torch.cuda.synchronize()
    # Two heads against the full (all rows, all columns) oracle.
    for b, h in ((0, 0), (1, 7)):
        q1, k1, q2, k2 = synth.head_inputs(w, b, h)
        g = synth.head_grad(w, b, h)
        ref = oracle.head_forward(q1, k1, q2, k2, w.scale1, w.scale2, True)
        err = np.abs(kl[b, h].cpu().numpy() - ref["kl"])
        assert np.all(err <= 2e-3 + 1e-2 * np.abs(ref["kl"]))
        assert np.abs(l1[b, h].cpu().numpy() - ref["lse1"]).max() <= 1e-3
        assert np.abs(l2[b, h].cpu().numpy() - ref["lse2"]).max() <= 1e-3
        for setting, dq, dk in (("student", dq2, dk2), ("teacher", dq1, dk1)):
            rq, rk = oracle.head_backward(q1, k1, q2, k2, w.scale1, w.scale2, True, g, setting)
            check_grad(f"4K ({b},{h}) dQ {setting}", w, dq[b, h].float().cpu().numpy(), rq, per_head_axis=False)
            check_grad(f"4K ({b},{h}) dK {setting}", w, dk[b, h].float().cpu().numpy(), rk, per_head_axis=False)
    check_sampled_backward(w, dq2, dk2, "student", t=t)
    check_sampled_backward(w, dq1, dk1, "teacher", t=t)


@pytest.mark.parametrize("causal", [True, False])
def test_16k_forward_and_splitk(gpu_lib, store, causal):
    w0, t = inputs(store, "n16k_h32_d128_corr05")
    w = w0.with_(causal=causal)
    say(f"[full] 16K forward causal={causal}")
    kl, l1, l2 = gpu_lib.skl_forward(t["q1"], t["k1"], t["q2"], t["k2"], w.scale1, w.scale2, causal)
    torch.cuda.synchronize()
    check_sampled_forward(w, kl, l1, l2)
    for splits in (2, 4, 8):
        say(f"[full] 16K split-K {splits} causal={causal}")
        ws, n = gpu_lib.skl_forward_splitk(t["q1"], t["k1"], t["q2"], t["k2"], w.scale1, w.scale2, causal, splits)
        skl_kl, s1, s2 = gpu_lib.skl_reduce(ws, n, w.B, w.H, w.NQ)
        torch.cuda.synchronize()
        for a, b_ in ((skl_kl, kl), (s1, l1), (s2, l2)):
            assert torch.allclose(a, b_, rtol=2e-5, atol=2e-5)
        check_sampled_forward(w, skl_kl, s1, s2, rows_seed=splits)


@pytest.mark.parametrize("causal", [True, False])
def test_16k_backward_full_head(gpu_lib, store, causal):
    """Both backward settings at 16K x 16K, 32 heads, through the student and
    teacher calls and through one joint call: every row of dQ and every key
    column of dK of one head against the oracle (early key columns walk every
    query tile, late ones only the diagonal), sampled rows of two more heads,
    and sum_j dK_j = 0 for all heads."""
    w0, t = inputs(store, "n16k_h32_d128_corr05")
    w = w0.with_(causal=causal)
    kl, l1, l2 = gpu_lib.skl_forward(t["q1"], t["k1"], t["q2"], t["k2"], w.scale1, w.scale2, causal)
    b, h = 0, w.H - 1
    q1, k1, q2, k2 = synth.head_inputs(w, b, h)
    g = synth.head_grad(w, b, h)
    ref = {s_: oracle.head_backward(q1, k1, q2, k2, w.scale1, w.scale2, causal, g, s_) for s_ in ("student", "teacher")}
    for setting, dq, dk in backward_calls(gpu_lib, t, w, kl, l1, l2, causal):
        rq, rk = ref[setting]
        check_grad(f"16K ({b},{h}) dQ {setting} causal={causal}", w, dq[b, h].float().cpu().numpy(), rq,
                   per_head_axis=False)
        check_grad(f"16K ({b},{h}) dK {setting} causal={causal}", w, dk[b, h].float().cpu().numpy(), rk,
                   per_head_axis=False)
        check_sampled_backward(w, dq, dk, setting, t=t)


def test_causal_64k_forward_student_teacher(gpu_lib, store):
    w, t = inputs(store, "causal_64k_h32_d128_q1x4")
    say("[full] causal 64K forward")
    kl, l1, l2 = gpu_lib.skl_forward(t["q1"], t["k1"], t["q2"], t["k2"], w.scale1, w.scale2, True)
    torch.cuda.synchronize()
    check_sampled_forward(w, kl, l1, l2)
    say("[full] causal 64K student backward")
    dq, dk = gpu_lib.skl_backward_student(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, t["g"],
                                          w.scale1, w.scale2, True)
    torch.cuda.synchronize()
    check_sampled_backward(w, dq, dk, "student", t=t)
    del dq, dk
    say("[full] causal 64K teacher backward")
    dq, dk = gpu_lib.skl_backward_teacher(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, kl, t["g"],
                                          w.scale1, w.scale2, True)
    torch.cuda.synchronize()
    check_sampled_backward(w, dq, dk, "teacher", early_cols_head=(0, 5), t=t)


def test_causal_64k_joint_backward(gpu_lib, store):
    """The joint call bench.py times by default, at its full size: sampled
    rows and trailing key columns of both settings, the first key columns of
    one head (teacher; the two dK products share the kernel's loop), and
    sum_j dK_j = 0 for every head."""
    w, t = inputs(store, "causal_64k_h32_d128_q1x4")
    kl, l1, l2 = gpu_lib.skl_forward(t["q1"], t["k1"], t["q2"], t["k2"], w.scale1, w.scale2, True)
    say("[full] causal 64K joint backward")
    dq1, dk1, dq2, dk2 = gpu_lib.skl_backward_joint(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, kl, t["g"],
                                                    w.scale1, w.scale2, True)
    torch.cuda.synchronize()
    check_sampled_backward(w, dq1, dk1, "teacher", early_cols_head=(0, 9), t=t)
    del dq1, dk1
    check_sampled_backward(w, dq2, dk2, "student", t=t)


def test_noncausal_64k_forward_and_joint_backward(gpu_lib, store):
    """The same 64K x 64K inputs without the mask, as bench.py's unmasked leg
    times them: the forward and the joint call on sampled rows, and for every
    head sum_j dK_j = 0 and the dQ / dK identity.  (Key columns against the
    oracle would need every row's full softmax: about ten minutes of the
    oracle per head at this size, so the 16K whole-head test covers dK
    columns without the mask.)"""
    w, t = inputs(store, "causal_64k_h32_d128_q1x4")
    wn = w.with_(causal=False)  # same seed, same tensors
    say("[full] non-causal 64K forward")
    kl, l1, l2 = gpu_lib.skl_forward(t["q1"], t["k1"], t["q2"], t["k2"], wn.scale1, wn.scale2, False)
    torch.cuda.synchronize()
    check_sampled_forward(wn, kl, l1, l2, rows_seed=3)
    say("[full] non-causal 64K joint backward")
    dq1, dk1, dq2, dk2 = gpu_lib.skl_backward_joint(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, kl, t["g"],
                                                    wn.scale1, wn.scale2, False)
    torch.cuda.synchronize()
    check_sampled_backward(wn, dq1, dk1, "teacher", t=t)
    del dq1, dk1
    check_sampled_backward(wn, dq2, dk2, "student", t=t)


def test_causal_128k_indexer_student(gpu_lib, store):
    w, t = inputs(store, "causal_128k_h8_d128_d64")
    say("[full] causal 128K (d1=128, d2=64) forward")
    kl, l1, l2 = gpu_lib.skl_forward(t["q1"], t["k1"], t["q2"], t["k2"], w.scale1, w.scale2, True)
    torch.cuda.synchronize()
    check_sampled_forward(w, kl, l1, l2)
    say("[full] causal 128K student backward")
    dq, dk = gpu_lib.skl_backward_student(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, t["g"],
                                          w.scale1, w.scale2, True)
    torch.cuda.synchronize()
    check_sampled_backward(w, dq, dk, "student", t=t)
    del dq, dk
    say("[full] causal 128K joint backward")
    dq1, dk1, dq2, dk2 = gpu_lib.skl_backward_joint(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, kl, t["g"],
                                                    w.scale1, w.scale2, True)
    torch.cuda.synchronize()
    check_sampled_backward(w, dq1, dk1, "teacher", t=t)
    check_sampled_backward(w, dq2, dk2, "student", t=t)


@pytest.mark.parametrize("name", ["causal_256k_h4_d128", "causal_512k_h2_d128"])
def test_long_context_forward_and_both_backward(gpu_lib, store, name):
    """256K and 512K contexts on one GPU: sampled rows, trailing key columns
    and sum_j dK_j = 0, for the forward and both backward settings."""
    w, t = inputs(store, name)
    say(f"[full] {name} forward")
    kl, l1, l2 = gpu_lib.skl_forward(t["q1"], t["k1"], t["q2"], t["k2"], w.scale1, w.scale2, True)
    torch.cuda.synchronize()
    check_sampled_forward(w, kl, l1, l2)
    for setting, dq, dk in backward_calls(gpu_lib, t, w, kl, l1, l2, True):
        check_sampled_backward(w, dq, dk, setting, t=t)


def test_query_chunk_of_long_sequence(gpu_lib, store):
    """1024 queries at the end of a 256K causal sequence (bottom-right
    alignment): few query tiles, so the recommended split count is > 1; the
    split-K forward agrees with the plain one and both match the oracle."""
    w, t = inputs(store, "chunk_1k_of_256k_h8_d128")
    say("[full] 1K-query chunk of 256K: forward")
    kl, l1, l2 = gpu_lib.skl_forward(t["q1"], t["k1"], t["q2"], t["k2"], w.scale1, w.scale2, True)
    torch.cuda.synchronize()
    check_sampled_forward(w, kl, l1, l2)
    splits = gpu_lib.skl_recommended_splits(t["q1"], t["k1"], t["q2"], t["k2"], True)
    assert splits > 1
    say(f"[full] 1K-query chunk of 256K: split-K {splits}")
    ws, n = gpu_lib.skl_forward_splitk(t["q1"], t["k1"], t["q2"], t["k2"], w.scale1, w.scale2, True, splits)
    skl_kl, s1, s2 = gpu_lib.skl_reduce(ws, n, w.B, w.H, w.NQ)
    torch.cuda.synchronize()
    for a, b_ in ((skl_kl, kl), (s1, l1), (s2, l2)):
        assert torch.allclose(a, b_, rtol=2e-5, atol=2e-5)
    for setting in ("student", "teacher"):
        say(f"[full] 1K-query chunk of 256K: {setting} backward")
        if setting == "student":
            dq, dk = gpu_lib.skl_backward_student(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, t["g"],
                                                  w.scale1, w.scale2, True)
        else:
            dq, dk = gpu_lib.skl_backward_teacher(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, kl, t["g"],
                                                  w.scale1, w.scale2, True)
        torch.cuda.synchronize()
        check_sampled_backward(w, dq, dk, setting, t=t)
        del dq, dk
