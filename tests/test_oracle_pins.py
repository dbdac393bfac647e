"""Pins of the float64 oracle to facts other than itself.

Each test compares the oracle with something the mathematics fixes: exact
invariants, closed forms, a library routine, brute force in scalar Python, or
finite differences.  Together they are meant to catch a dropped term, a wrong
sign, a wrong index or mask, or a transposed operand anywhere in the oracle.
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle
from attention_kl_divergence_skl_amd import synth


def _rand(rng, n, d, amp=1.0):
    return amp * rng.standard_normal((n, d))


def _inputs(seed, nq, nk, d1, d2, amp1=1.0, amp2=1.0):
    rng = np.random.default_rng(seed)
    return (_rand(rng, nq, d1, amp1), _rand(rng, nk, d1), _rand(rng, nq, d2, amp2), _rand(rng, nk, d2))


SHAPES = [(1, 1, 1, 1), (3, 5, 2, 2), (7, 7, 4, 3), (13, 13, 8, 8), (5, 11, 4, 4), (40, 65, 6, 5)]


# ------------------------------------------------------------ invariants ----

@pytest.mark.parametrize("causal", [False, True])
def test_identical_distributions_give_zero_kl_exactly(causal):
    w = synth.Workload("t", 1, 2, 70, 70, 16, 16, "bf16", causal, 0.25, 0.25,
                       synth.Recipe("identical", amp1=3.0), seed=7)
    for h in range(2):
        q1, k1, q2, k2 = synth.head_inputs(w, 0, h)
        r = oracle.head_forward(q1, k1, q2, k2, 0.25, 0.25, causal)
        assert np.all(r["kl"] == 0.0)
        assert np.array_equal(r["lse1"], r["lse2"])


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("causal", [False, True])
def test_kl_is_nonnegative(seed, causal):
    nq, nk = (30, 41) if causal else (37, 23)
    q1, k1, q2, k2 = _inputs(seed, nq, nk, 5, 7, amp1=2.0)
    r = oracle.head_forward(q1, k1, q2, k2, 0.7, 0.4, causal)
    assert np.all(r["kl"] >= -1e-12)
    assert np.all(r["kl"][np.abs(r["kl"]) > 0] > 0)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_changes_lse_only(causal):
    """Adding one vector v to every key multiplies each softmax row by a
    constant: KL is unchanged and LSE moves by scale * <q_i, v>."""
    q1, k1, q2, k2 = _inputs(3, 9, 12, 4, 6)
    rng = np.random.default_rng(11)
    v1, v2 = rng.standard_normal(4), rng.standard_normal(6)
    base = oracle.head_forward(q1, k1, q2, k2, 0.9, 0.6, causal)
    shifted = oracle.head_forward(q1, k1 + v1, q2, k2 + v2, 0.9, 0.6, causal)
    np.testing.assert_allclose(shifted["kl"], base["kl"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(shifted["lse1"], base["lse1"] + 0.9 * (q1 @ v1), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(shifted["lse2"], base["lse2"] + 0.6 * (q2 @ v2), rtol=1e-12, atol=1e-12)


def test_shifted_copy_has_zero_kl_but_large_lse_gap():
    """Q2 = Q1 and K2 = K1 + v: P2 == P1 although S2 - S1 is large."""
    q1, k1, _, _ = _inputs(5, 16, 16, 8, 8)
    v = 25.0 * np.ones(8)
    r = oracle.head_forward(q1, k1, q1, k1 + v, 0.5, 0.5, False)
    np.testing.assert_allclose(r["kl"], 0.0, atol=1e-11)
    assert np.all(np.abs(r["lse2"] - r["lse1"]) > 1.0)


def test_joint_key_permutation_invariance():
    q1, k1, q2, k2 = _inputs(8, 10, 17, 5, 5)
    perm = np.random.default_rng(2).permutation(17)
    a = oracle.head_forward(q1, k1, q2, k2, 0.8, 0.8, False)
    b = oracle.head_forward(q1, k1[perm], q2, k2[perm], 0.8, 0.8, False)
    for k in a:
        np.testing.assert_allclose(b[k], a[k], rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------- closed forms ----

@pytest.mark.parametrize("causal,nq,nk", [(False, 12, 31), (True, 20, 20), (True, 9, 25)])
def test_uniform_teacher_closed_form(causal, nq, nk):
    """Q1 = 0 makes P1 uniform over the n_i allowed keys of row i, so
    LSE1 = log n_i and KL = -log n_i - mean_allowed(S2) + LSE2."""
    _, k1, q2, k2 = _inputs(4, nq, nk, 6, 6)
    q1 = np.zeros((nq, 6))
    r = oracle.head_forward(q1, k1, q2, k2, 0.3, 0.45, causal)
    off = nk - nq
    for i in range(nq):
        n_i = (i + off + 1) if causal else nk
        s2 = 0.45 * (k2[:n_i] @ q2[i])
        lse2 = scipy.special.logsumexp(s2)
        assert r["lse1"][i] == pytest.approx(math.log(n_i), rel=1e-14, abs=1e-14)
        assert r["lse2"][i] == pytest.approx(lse2, rel=1e-13, abs=1e-13)
        assert r["kl"][i] == pytest.approx(-math.log(n_i) - s2.mean() + lse2, rel=1e-11, abs=1e-12)


def test_two_key_bernoulli_closed_form():
    """With two keys each softmax row is a Bernoulli(p) with p = sigmoid(s0 - s1)."""
    q1, k1, q2, k2 = _inputs(6, 25, 2, 3, 5, amp1=2.0)
    r = oracle.head_forward(q1, k1, q2, k2, 1.1, 0.7, False)
    s1, s2 = 1.1 * q1 @ k1.T, 0.7 * q2 @ k2.T
    p = scipy.special.expit(s1[:, 0] - s1[:, 1])
    q = scipy.special.expit(s2[:, 0] - s2[:, 1])
    expect = p * np.log(p / q) + (1 - p) * np.log((1 - p) / (1 - q))
    np.testing.assert_allclose(r["kl"], expect, rtol=1e-10, atol=1e-13)


@pytest.mark.parametrize("nq,nk", [(10, 10), (4, 9)])
def test_causal_first_row(nq, nk):
    """Bottom-right causal alignment: row 0 sees keys 0..N_K-N_Q.  With one key
    both distributions are a point mass: KL = 0 and LSE = the single logit."""
    q1, k1, q2, k2 = _inputs(9, nq, nk, 4, 4)
    r = oracle.head_forward(q1, k1, q2, k2, 0.5, 0.25, True)
    off = nk - nq
    s1 = 0.5 * k1[:off + 1] @ q1[0]
    s2 = 0.25 * k2[:off + 1] @ q2[0]
    assert r["lse1"][0] == pytest.approx(scipy.special.logsumexp(s1), rel=1e-13)
    assert r["lse2"][0] == pytest.approx(scipy.special.logsumexp(s2), rel=1e-13)
    if off == 0:
        assert r["kl"][0] == 0.0
        assert r["lse1"][0] == pytest.approx(s1[0], rel=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_lse_matches_scipy_logsumexp(causal):
    q1, k1, q2, k2 = _inputs(10, 33, 47, 8, 8, amp1=6.0)
    r = oracle.head_forward(q1, k1, q2, k2, 0.35, 0.35, causal)
    off = 47 - 33
    for i in range(33):
        n = (i + off + 1) if causal else 47
        assert r["lse1"][i] == pytest.approx(scipy.special.logsumexp(0.35 * k1[:n] @ q1[i]), rel=1e-13)
        assert r["lse2"][i] == pytest.approx(scipy.special.logsumexp(0.35 * k2[:n] @ q2[i]), rel=1e-13)


# ----------------------------------------------------- brute force (tiny) ----

def _brute(q1, k1, q2, k2, s1c, s2c, causal):
    nq, nk = len(q1), len(k1)
    kl, l1s, l2s = [], [], []
    for i in range(nq):
        keys = [j for j in range(nk) if (not causal) or j <= i + nk - nq]
        s1 = [s1c * sum(float(a) * float(b) for a, b in zip(q1[i], k1[j])) for j in keys]
        s2 = [s2c * sum(float(a) * float(b) for a, b in zip(q2[i], k2[j])) for j in keys]
        z1 = sum(math.exp(x) for x in s1)
        z2 = sum(math.exp(x) for x in s2)
        p1 = [math.exp(x) / z1 for x in s1]
        p2 = [math.exp(x) / z2 for x in s2]
        kl.append(sum(a * math.log(a / b) for a, b in zip(p1, p2)))
        l1s.append(math.log(z1))
        l2s.append(math.log(z2))
    return np.array(kl), np.array(l1s), np.array(l2s)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_forward_matches_scalar_brute_force(shape, causal):
    nq, nk, d1, d2 = shape
    if causal and nq > nk:
        pytest.skip("causal needs N_Q <= N_K")
    q1, k1, q2, k2 = _inputs(sum(shape), nq, nk, d1, d2)
    kl, lse1, lse2 = _brute(q1, k1, q2, k2, 0.6, 0.8, causal)
    r = oracle.head_forward(q1, k1, q2, k2, 0.6, 0.8, causal)
    np.testing.assert_allclose(r["kl"], kl, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(r["lse1"], lse1, rtol=1e-12)
    np.testing.assert_allclose(r["lse2"], lse2, rtol=1e-12)


# --------------------------------------------- the pages' online rewrite ----

@pytest.mark.parametrize("block_k,splits", [(1, 1), (3, 1), (16, 1), (64, 1), (5, 2), (8, 3), (4, 7)])
@pytest.mark.parametrize("causal,nq,nk", [(False, 29, 29), (True, 29, 29), (True, 10, 37), (False, 13, 50)])
def test_online_rewrite_matches_definition(block_k, splits, causal, nq, nk):
    q1, k1, q2, k2 = _inputs(block_k * 7 + splits, nq, nk, 6, 4, amp1=3.0)
    ref = oracle.head_forward(q1, k1, q2, k2, 0.5, 0.9, causal)
    on = oracle.online_forward(q1, k1, q2, k2, 0.5, 0.9, causal, block_k=block_k, splits=splits)
    for k in ref:
        np.testing.assert_allclose(on[k], ref[k], rtol=1e-10, atol=1e-10)


# --------------------------------------------------------------- gradients ----

def _loss(q1, k1, q2, k2, s1, s2, causal, g):
    return float(np.dot(g, oracle.head_forward(q1, k1, q2, k2, s1, s2, causal)["kl"]))


@pytest.mark.parametrize("setting", ["student", "teacher"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1), (2, 3, 2, 1), (5, 5, 4, 2), (8, 13, 3, 4), (13, 13, 8, 8)])
def test_gradients_match_finite_differences(setting, causal, shape):
    nq, nk, d1, d2 = shape
    q1, k1, q2, k2 = _inputs(100 + sum(shape), nq, nk, d1, d2, amp1=1.5)
    g = np.random.default_rng(sum(shape)).standard_normal(nq)
    sc1, sc2 = 0.7, 0.55
    dq, dk = oracle.head_backward(q1, k1, q2, k2, sc1, sc2, causal, g, setting)
    args = [q1, k1, q2, k2]
    iq, ik = (2, 3) if setting == "student" else (0, 1)
    for idx, analytic in ((iq, dq), (ik, dk)):
        num = np.zeros_like(args[idx])
        for pos in np.ndindex(*args[idx].shape):
            x0 = args[idx][pos]
            h = 1e-6 * max(1.0, abs(x0))
            a = [x.copy() for x in args]
            a[idx][pos] = x0 + h
            fp = _loss(*a, sc1, sc2, causal, g)
            a[idx][pos] = x0 - h
            fm = _loss(*a, sc1, sc2, causal, g)
            num[pos] = (fp - fm) / (2 * h)
        err = np.linalg.norm(analytic - num) / max(np.linalg.norm(num), 1e-30)
        assert err <= 1e-6 or np.linalg.norm(analytic - num) < 1e-10


@pytest.mark.parametrize("causal,nq,nk", [(False, 23, 31), (True, 26, 26), (True, 17, 30)])
def test_gradients_match_torch_autograd(causal, nq, nk):
    torch = pytest.importorskip("torch")
    q1, k1, q2, k2 = _inputs(55, nq, nk, 5, 7, amp1=2.5)
    g = np.random.default_rng(1).standard_normal(nq)
    sc1, sc2 = 0.45, 0.8
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q1, k1, q2, k2)]
    allow = torch.tensor(oracle.allowed_keys(np.arange(nq), nq, nk, causal))
    # A finite fill far below exp's underflow keeps autograd free of inf - inf.
    s1 = (sc1 * t[0] @ t[1].T).masked_fill(~allow, -1e4)
    s2 = (sc2 * t[2] @ t[3].T).masked_fill(~allow, -1e4)
    lp1 = torch.log_softmax(s1, dim=1)
    lp2 = torch.log_softmax(s2, dim=1)
    terms = torch.where(allow, lp1.exp() * (lp1 - lp2), torch.zeros((), dtype=torch.float64))
    loss = (torch.tensor(g) * terms.sum(dim=1)).sum()
    loss.backward()
    dq2, dk2 = oracle.head_backward(q1, k1, q2, k2, sc1, sc2, causal, g, "student")
    dq1, dk1 = oracle.head_backward(q1, k1, q2, k2, sc1, sc2, causal, g, "teacher")
    np.testing.assert_allclose(dq1, t[0].grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk1, t[1].grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dq2, t[2].grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk2, t[3].grad.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("setting", ["student", "teacher"])
@pytest.mark.parametrize("causal", [False, True])
def test_key_gradients_sum_to_zero(setting, causal):
    """Each row of dS sums to zero (softmax rows sum to one), so the key
    gradients of one head sum to the zero vector."""
    q1, k1, q2, k2 = _inputs(21, 30, 30, 6, 6, amp1=2.0)
    g = np.random.default_rng(3).standard_normal(30)
    _, dk = oracle.head_backward(q1, k1, q2, k2, 0.5, 0.5, causal, g, setting)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12 * max(1.0, np.abs(dk).max()))


def test_equal_queries_and_keys_give_zero_key_gradient():
    """All keys equal -> every softmax row is uniform in both settings, so
    dS = 0 for the student and for the teacher alike."""
    rng = np.random.default_rng(4)
    k = np.tile(rng.standard_normal(4), (9, 1))
    q1, q2 = rng.standard_normal((6, 4)), rng.standard_normal((6, 4))
    g = rng.standard_normal(6)
    for setting in ("student", "teacher"):
        dq, dk = oracle.head_backward(q1, k, q2, k, 0.5, 0.5, False, g, setting)
        np.testing.assert_allclose(dk, 0.0, atol=1e-14)
        np.testing.assert_allclose(dq, 0.0, atol=1e-14)


@pytest.mark.parametrize("setting", ["student", "teacher"])
@pytest.mark.parametrize("causal,nq,nk", [(False, 300, 280), (True, 290, 290), (True, 270, 300)])
def test_sampled_rows_and_columns_match_full_backward(setting, causal, nq, nk):
    q1, k1, q2, k2 = _inputs(77, nq, nk, 4, 4)
    g = np.random.default_rng(5).standard_normal(nq)
    dq, dk = oracle.head_backward(q1, k1, q2, k2, 0.5, 0.6, causal, g, setting)
    rows = np.array([0, 1, 63, 257, nq - 1])
    cols = np.array([nk - 1, nk - 40, nk - 257, 3])
    np.testing.assert_allclose(oracle.head_dq_rows(q1, k1, q2, k2, 0.5, 0.6, causal, g, setting, rows),
                               dq[rows], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(oracle.head_dk_cols(q1, k1, q2, k2, 0.5, 0.6, causal, g, setting, cols),
                               dk[cols], rtol=1e-11, atol=1e-15)


def test_teacher_gradient_is_finite_when_probabilities_underflow():
    """Logit gaps of hundreds of nats: P underflows to exactly 0 for most keys
    and log P would be -inf; the log-ratio from logits keeps everything finite."""
    q1, k1, q2, k2 = _inputs(31, 16, 16, 8, 8, amp1=60.0, amp2=40.0)
    g = np.ones(16)
    for causal in (False, True):
        r = oracle.head_forward(q1, k1, q2, k2, 1.0, 1.0, causal)
        assert np.all(np.isfinite(r["kl"]))
        for setting in ("student", "teacher"):
            dq, dk = oracle.head_backward(q1, k1, q2, k2, 1.0, 1.0, causal, g, setting)
            assert np.all(np.isfinite(dq)) and np.all(np.isfinite(dk))


# ------------------------------------------------ batched [B, H, N, d] calls ----
#
# oracle.forward / oracle.backward loop over (batch, head) and call the
# per-head functions.  These pins check the loop itself: every (b, h) slice of
# the output must come from the same (b, h) slices of all four inputs (and of
# g), with scale1 on the (Q1, K1) side and scale2 on the (Q2, K2) side.  The
# shapes make every axis distinguishable: B != H, N_Q != N_K, d1 != d2 and
# unequal scales.

BATCHED_SHAPE = dict(B=2, H=3, nq=5, nk=7, d1=3, d2=2)
BATCHED_SCALES = (0.9, 0.35)


def _batched_inputs(seed):
    s = BATCHED_SHAPE
    rng = np.random.default_rng(seed)
    q1 = 1.5 * rng.standard_normal((s["B"], s["H"], s["nq"], s["d1"]))
    k1 = rng.standard_normal((s["B"], s["H"], s["nk"], s["d1"]))
    q2 = rng.standard_normal((s["B"], s["H"], s["nq"], s["d2"]))
    k2 = rng.standard_normal((s["B"], s["H"], s["nk"], s["d2"]))
    g = rng.standard_normal((s["B"], s["H"], s["nq"]))
    return q1, k1, q2, k2, g


@pytest.mark.parametrize("causal", [False, True])
def test_batched_forward_matches_brute_force_per_head(causal):
    q1, k1, q2, k2, _ = _batched_inputs(41)
    sc1, sc2 = BATCHED_SCALES
    r = oracle.forward(q1, k1, q2, k2, sc1, sc2, causal)
    B, H = q1.shape[:2]
    for k in ("kl", "lse1", "lse2"):
        assert r[k].shape == (B, H, q1.shape[2])
    for b in range(B):
        for h in range(H):
            kl, lse1, lse2 = _brute(q1[b, h], k1[b, h], q2[b, h], k2[b, h], sc1, sc2, causal)
            np.testing.assert_allclose(r["kl"][b, h], kl, rtol=1e-10, atol=1e-13)
            np.testing.assert_allclose(r["lse1"][b, h], lse1, rtol=1e-12)
            np.testing.assert_allclose(r["lse2"][b, h], lse2, rtol=1e-12)


def _batched_brute_loss(q1, k1, q2, k2, sc1, sc2, causal, g):
    """sum over (b, h, i) of g[b, h, i] * KL[b, h, i], all in scalar Python."""
    total = 0.0
    for b in range(q1.shape[0]):
        for h in range(q1.shape[1]):
            kl, _, _ = _brute(q1[b, h], k1[b, h], q2[b, h], k2[b, h], sc1, sc2, causal)
            total += float(np.dot(g[b, h], kl))
    return total


@pytest.mark.parametrize("setting", ["student", "teacher"])
@pytest.mark.parametrize("causal", [False, True])
def test_batched_backward_matches_finite_differences(setting, causal):
    """Central differences of the scalar brute-force loss with respect to
    every element of every head: a gradient written to the wrong head, or
    computed from another head's inputs or g, fails here."""
    q1, k1, q2, k2, g = _batched_inputs(42)
    sc1, sc2 = BATCHED_SCALES
    dq, dk = oracle.backward(q1, k1, q2, k2, sc1, sc2, causal, g, setting)
    args = [q1, k1, q2, k2]
    iq, ik = (2, 3) if setting == "student" else (0, 1)
    assert dq.shape == args[iq].shape and dk.shape == args[ik].shape
    for idx, analytic in ((iq, dq), (ik, dk)):
        num = np.zeros_like(args[idx])
        for pos in np.ndindex(*args[idx].shape):
            x0 = args[idx][pos]
            h = 1e-6 * max(1.0, abs(x0))
            a = [x.copy() for x in args]
            a[idx][pos] = x0 + h
            fp = _batched_brute_loss(*a, sc1, sc2, causal, g)
            a[idx][pos] = x0 - h
            fm = _batched_brute_loss(*a, sc1, sc2, causal, g)
            num[pos] = (fp - fm) / (2 * h)
        err = np.linalg.norm(analytic - num) / max(np.linalg.norm(num), 1e-30)
        assert err <= 1e-6, f"{setting} input {idx}: relative error {err:.3e}"
        # Per head as well, so that one head's error cannot hide in the total.
        for b in range(num.shape[0]):
            for hh in range(num.shape[1]):
                eh = np.linalg.norm(analytic[b, hh] - num[b, hh])
                assert eh <= 1e-6 * max(np.linalg.norm(num[b, hh]), 1e-4), (setting, idx, b, hh, eh)
