"""GPU parity: the HIP path through the C ABI against the float64 oracle, on
seeded inputs the oracle finishes in seconds.  Shapes span several tiles and
ragged tails; edge cases cover single rows, N_Q != N_K, unequal head dims,
strided layouts, identical and uniform distributions and underflowing
probabilities."""
import numpy as np
import pytest
import torch

import oracle
from attention_kl_divergence_skl_amd import synth
from tests.gpu_util import (TOL, check_grad, check_rows, gpu_forward, grad_to_np, oracle_backward,
                            oracle_forward, say, to_device)

pytestmark = pytest.mark.gpu

S128 = 1 / np.sqrt(128)
S64 = 1 / np.sqrt(64)


def W(name, B, H, NQ, NK, d1, d2, dtype, causal, recipe=synth.Recipe("iid"), grad="random", seed=1,
      scale1=None, scale2=None):
    return synth.Workload(name, B, H, NQ, NK, d1, d2, dtype, causal,
                          scale1 if scale1 is not None else 1 / np.sqrt(d1),
                          scale2 if scale2 is not None else 1 / np.sqrt(d2), recipe, grad, seed)


CASES = [
    synth.WORKLOADS["tiny_f32_n256_d64"],
    W("f32_ragged_causal", 1, 2, 200, 200, 64, 64, "f32", True),
    W("f32_d128_noncausal", 2, 1, 130, 190, 128, 128, "f32", False),
    W("bf16_ragged_causal", 1, 2, 300, 300, 128, 128, "bf16", True, synth.Recipe("corr", noise=0.3)),
    W("bf16_ragged_noncausal", 2, 2, 257, 257, 128, 128, "bf16", False, synth.Recipe("corr", noise=0.5)),
    W("bf16_nq_lt_nk_causal", 1, 2, 100, 333, 128, 128, "bf16", True),
    W("bf16_nq_ne_nk_noncausal", 1, 1, 333, 77, 128, 128, "bf16", False),
    W("bf16_d128_d64_causal", 1, 2, 290, 290, 128, 64, "bf16", True),
    W("bf16_d64_d128_noncausal", 1, 2, 150, 250, 64, 128, "bf16", False),
    W("bf16_d64_d64_causal", 2, 1, 255, 255, 64, 64, "bf16", True, synth.Recipe("iid", amp1=4.0)),
    W("bf16_single_row", 1, 1, 1, 1, 128, 128, "bf16", True),
    W("bf16_one_query_many_keys", 1, 1, 1, 517, 128, 64, "bf16", False),
    W("bf16_n17", 1, 3, 17, 17, 128, 128, "bf16", True),
    # Tile-aligned and half-aligned shapes: the backward separates the steps
    # that reach the causal diagonal or a ragged edge from mask-free ones, so
    # these pin each combination of aligned / ragged N_Q and N_K.
    W("bf16_aligned_causal", 1, 2, 512, 512, 128, 128, "bf16", True, synth.Recipe("corr", noise=0.3)),
    W("f32_aligned_causal", 1, 1, 384, 384, 64, 64, "f32", True),
    W("bf16_nq_aligned_nk_ragged_causal", 1, 2, 256, 333, 128, 128, "bf16", True),
    W("bf16_nq_ragged_nk_aligned_causal", 1, 2, 200, 512, 128, 64, "bf16", True),
    W("bf16_nq_aligned_nk_ragged_noncausal", 1, 2, 384, 200, 64, 128, "bf16", False),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_forward_matches_oracle(gpu_lib, w):
    say(f"[forward] {w.name}")
    x, t = to_device(w)
    got, _ = gpu_forward(gpu_lib, w, t)
    check_rows(w.name, w, got, oracle_forward(w, x))


@pytest.mark.parametrize("algo", ["split", "split_no_ws", "fused_atomic"])
@pytest.mark.parametrize("setting", ["student", "teacher"])
@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_backward_matches_oracle(gpu_lib, w, setting, algo):
    """split: dQ over key ranges whenever the query tiles are few (all of
    these shapes); split_no_ws: the same kernels with dQ over all keys."""
    say(f"[backward {setting} {algo}] {w.name}")
    x, t = to_device(w)
    _, (kl, l1, l2) = gpu_forward(gpu_lib, w, t)
    ws = torch.empty(0, dtype=torch.float32, device="cuda") if algo == "split_no_ws" else None
    a = "split" if algo == "split_no_ws" else algo
    if setting == "student":
        dq, dk = gpu_lib.skl_backward_student(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, t["g"],
                                              w.scale1, w.scale2, w.causal, algo=a, ws=ws)
    else:
        dq, dk = gpu_lib.skl_backward_teacher(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, kl, t["g"],
                                              w.scale1, w.scale2, w.causal, algo=a, ws=ws)
    torch.cuda.synchronize()
    rq, rk = oracle_backward(w, x, setting)
    check_grad(f"{w.name} dQ ({setting})", w, grad_to_np(dq), rq)
    check_grad(f"{w.name} dK ({setting})", w, grad_to_np(dk), rk)


def test_strided_bnhd_layout(gpu_lib):
    w = W("bf16_bnhd", 2, 3, 190, 190, 128, 64, "bf16", True)
    say(f"[layout bnhd] {w.name}")
    x, t = to_device(w, layout="bnhd")
    assert not t["q1"].is_contiguous()
    got, (kl, l1, l2) = gpu_forward(gpu_lib, w, t)
    check_rows(w.name, w, got, oracle_forward(w, x))
    dq, dk = gpu_lib.skl_backward_student(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, t["g"],
                                          w.scale1, w.scale2, w.causal)
    dq1, dk1 = gpu_lib.skl_backward_teacher(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, kl, t["g"],
                                            w.scale1, w.scale2, w.causal)
    none = torch.empty(0, dtype=torch.float32, device="cuda")
    joint = gpu_lib.skl_backward_joint(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, kl, t["g"],
                                       w.scale1, w.scale2, w.causal, ws=none)
    torch.cuda.synchronize()
    assert dq.stride() == t["q2"].stride() and dk.stride() == t["k2"].stride()
    for got_, ref_ in zip(joint, (t["q1"], t["k1"], t["q2"], t["k2"])):
        assert got_.stride() == ref_.stride()
    rq, rk = oracle_backward(w, x, "student")
    check_grad("bnhd dQ2", w, grad_to_np(dq), rq)
    check_grad("bnhd dK2", w, grad_to_np(dk), rk)
    check_grad("bnhd joint dQ2", w, grad_to_np(joint[2]), rq)
    check_grad("bnhd joint dK2", w, grad_to_np(joint[3]), rk)
    rq, rk = oracle_backward(w, x, "teacher")
    check_grad("bnhd dQ1", w, grad_to_np(dq1), rq)
    check_grad("bnhd dK1", w, grad_to_np(dk1), rk)
    check_grad("bnhd joint dQ1", w, grad_to_np(joint[0]), rq)
    check_grad("bnhd joint dK1", w, grad_to_np(joint[1]), rk)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_identical_inputs_give_zero_kl(gpu_lib, dtype, causal):
    w = W(f"identical_{dtype}", 1, 2, 200, 200, 64, 64, dtype, causal, synth.Recipe("identical", amp1=2.0))
    say(f"[identical] {w.name} causal={causal}")
    x, t = to_device(w)
    got, (kl, l1, l2) = gpu_forward(gpu_lib, w, t)
    assert np.all(got["kl"] == 0.0), "bitwise-equal logits must give KL == 0 exactly"
    assert np.array_equal(got["lse1"], got["lse2"])
    dq, dk = gpu_lib.skl_backward_student(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, t["g"],
                                          w.scale1, w.scale2, w.causal)
    torch.cuda.synchronize()
    assert float(dq.float().abs().max()) == 0.0 and float(dk.float().abs().max()) == 0.0


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_teacher_closed_form(gpu_lib, causal):
    """Q1 = 0: LSE1 = log n_i exactly in real arithmetic."""
    w = W("uniform_teacher", 1, 1, 160, 160, 128, 128, "bf16", causal, synth.Recipe("uniform1"))
    say(f"[uniform teacher] causal={causal}")
    x, t = to_device(w)
    got, _ = gpu_forward(gpu_lib, w, t)
    n = (np.arange(160) + 1) if causal else np.full(160, 160)
    np.testing.assert_allclose(got["lse1"][0, 0], np.log(n), atol=1e-5)
    check_rows(w.name, w, got, oracle_forward(w, x))


@pytest.mark.parametrize("causal", [False, True])
def test_underflowing_probabilities_stay_finite(gpu_lib, causal):
    """Logit gaps of hundreds of nats: P underflows in fp32; the teacher's
    log-ratio from logits must still give finite, oracle-matching gradients."""
    w = W("peaked", 1, 2, 192, 192, 64, 64, "bf16", causal, synth.Recipe("iid", amp1=60.0, amp2=30.0),
          scale1=1.0, scale2=1.0)
    say(f"[peaked] causal={causal}")
    x, t = to_device(w)
    got, (kl, l1, l2) = gpu_forward(gpu_lib, w, t)
    ref = oracle_forward(w, x)
    # Rows of several hundred nats: absolute floors scale with |KL|.
    check_rows(w.name, w, got, ref)
    for setting in ("student", "teacher"):
        if setting == "student":
            dq, dk = gpu_lib.skl_backward_student(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, t["g"],
                                                  w.scale1, w.scale2, w.causal)
        else:
            dq, dk = gpu_lib.skl_backward_teacher(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, kl, t["g"],
                                                  w.scale1, w.scale2, w.causal)
        torch.cuda.synchronize()
        rq, rk = oracle_backward(w, x, setting)
        check_grad(f"peaked dQ ({setting})", w, grad_to_np(dq), rq)
        check_grad(f"peaked dK ({setting})", w, grad_to_np(dk), rk)


@pytest.mark.parametrize("signs", ["mixed", "nonnegative"])
@pytest.mark.parametrize("setting", ["student", "teacher", "joint"])
def test_backward_zero_and_negative_row_gradients(gpu_lib, setting, signs):
    """Upstream gradients with exact zeros (every fifth row) and either mixed
    signs or none negative: the kernels fold log2 |g| into the exponents (a
    zero g into an exponent that underflows), apply the sign to the finished
    dQ rows, and to dS in the dK tiles that have a row with g < 0."""
    w = W(f"gsign_{signs}", 1, 2, 300, 300, 128, 64, "bf16", True, synth.Recipe("iid", amp1=2.0))
    say(f"[row gradients {signs}] {setting}")
    x, t = to_device(w)
    g = x["g"].copy()
    if signs == "nonnegative":
        g = np.abs(g)
    g[..., ::5] = 0.0
    x["g"] = g
    t["g"] = torch.from_numpy(g).cuda()
    _, (kl, l1, l2) = gpu_forward(gpu_lib, w, t)
    if setting == "joint":
        none = torch.empty(0, dtype=torch.float32, device="cuda")
        dq1, dk1, dq2, dk2 = gpu_lib.skl_backward_joint(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, kl, t["g"],
                                                        w.scale1, w.scale2, w.causal, ws=none)
        torch.cuda.synchronize()
        for st, dq, dk in (("teacher", dq1, dk1), ("student", dq2, dk2)):
            rq, rk = oracle_backward(w, x, st)
            dqn = grad_to_np(dq)
            assert np.all(dqn[..., ::5, :] == 0.0), "rows with g = 0 must get dQ = 0 exactly"
            check_grad(f"gsign joint dQ ({st}, {signs})", w, dqn, rq)
            check_grad(f"gsign joint dK ({st}, {signs})", w, grad_to_np(dk), rk)
        return
    if setting == "student":
        dq, dk = gpu_lib.skl_backward_student(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, t["g"],
                                              w.scale1, w.scale2, w.causal)
    else:
        dq, dk = gpu_lib.skl_backward_teacher(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, kl, t["g"],
                                              w.scale1, w.scale2, w.causal)
    torch.cuda.synchronize()
    rq, rk = oracle_backward(w, x, setting)
    dqn = grad_to_np(dq)
    assert np.all(dqn[..., ::5, :] == 0.0), "rows with g = 0 must get dQ = 0 exactly"
    check_grad(f"gsign dQ ({setting}, {signs})", w, dqn, rq)
    check_grad(f"gsign dK ({setting}, {signs})", w, grad_to_np(dk), rk)


@pytest.mark.parametrize("causal", [False, True])
def test_rising_logits_overtake_running_max(gpu_lib, causal):
    """Key norms grow along the key axis, so late keys overtake each row's
    running maximum by far more than 2^64 in base-2 terms: the forward must
    leave its kept-maximum sums for the exact update with new maxima and
    correction factors, many times per row.  (bf16 only: LSE reaches ~220
    nats here, where one fp32 ulp exceeds the fp32 LSE tolerance.)"""
    w = W("rising_bf16", 1, 2, 256, 640, 64, 64, "bf16", causal,
          synth.Recipe("iid", amp1=6.0, amp2=6.0, kramp=8.0))
    say(f"[rising logits] {w.name} causal={causal}")
    x, t = to_device(w)
    # The inputs really do that: base-2 logits of the first 32 keys against the row maximum.
    s1 = (x["q1"][0, 0].astype(np.float64) @ x["k1"][0, 0].astype(np.float64).T) * w.scale1 / np.log(2)
    if causal:
        s1 = np.where(np.arange(w.NK)[None, :] <= np.arange(w.NQ)[:, None] + (w.NK - w.NQ), s1, -np.inf)
    gap = s1.max(axis=1) - s1[:, :32].max(axis=1)
    assert np.mean(gap > 80) > 0.9, "recipe must move the row maximum far past the first block's"
    got, (kl, l1, l2) = gpu_forward(gpu_lib, w, t)
    check_rows(w.name, w, got, oracle_forward(w, x))
    dq, dk = gpu_lib.skl_backward_student(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, t["g"],
                                          w.scale1, w.scale2, w.causal)
    torch.cuda.synchronize()
    rq, rk = oracle_backward(w, x, "student")
    check_grad(f"{w.name} dQ2", w, grad_to_np(dq), rq)
    check_grad(f"{w.name} dK2", w, grad_to_np(dk), rk)


@pytest.mark.parametrize("splits", [2, 5])
@pytest.mark.parametrize("causal", [False, True])
def test_rising_logits_split_k(gpu_lib, splits, causal):
    """The rising-logits inputs through split-K + reduce: splits whose later
    blocks overtake the first block's maximum take the per-block exact update
    on the second pass, through the split's own partials."""
    w = W("rising_split", 1, 2, 256, 640, 64, 64, "bf16", causal,
          synth.Recipe("iid", amp1=6.0, amp2=6.0, kramp=8.0))
    say(f"[rising logits, split-K {splits}] causal={causal}")
    x, t = to_device(w)
    ws, n = gpu_lib.skl_forward_splitk(t["q1"], t["k1"], t["q2"], t["k2"], w.scale1, w.scale2, causal, splits)
    kl, l1, l2 = gpu_lib.skl_reduce(ws, n, w.B, w.H, w.NQ)
    torch.cuda.synchronize()
    got = {"kl": kl.cpu().numpy(), "lse1": l1.cpu().numpy(), "lse2": l2.cpu().numpy()}
    check_rows(f"rising split{splits}", w, got, oracle_forward(w, x))


@pytest.mark.parametrize("splits", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("causal", [False, True])
def test_splitk_matches_oracle_and_plain_forward(gpu_lib, splits, causal):
    w = W("splitk", 1, 3, 333, 700, 128, 64, "bf16", causal, synth.Recipe("iid", amp1=2.0))
    say(f"[split-K] splits={splits} causal={causal}")
    x, t = to_device(w)
    plain, _ = gpu_forward(gpu_lib, w, t)
    ws, n = gpu_lib.skl_forward_splitk(t["q1"], t["k1"], t["q2"], t["k2"], w.scale1, w.scale2, causal, splits)
    kl, l1, l2 = gpu_lib.skl_reduce(ws, n, w.B, w.H, w.NQ)
    torch.cuda.synchronize()
    got = {"kl": kl.cpu().numpy(), "lse1": l1.cpu().numpy(), "lse2": l2.cpu().numpy()}
    check_rows(f"split{splits}", w, got, oracle_forward(w, x))
    for k in got:
        np.testing.assert_allclose(got[k], plain[k], rtol=2e-5, atol=2e-5)


def test_low_occupancy_split_shape(gpu_lib):
    """Few query rows, long keys (non-causal): the shape split-K exists for."""
    w = W("low_occupancy", 1, 1, 256, 16384, 128, 128, "bf16", False, synth.Recipe("corr", noise=0.5))
    say("[split-K] low occupancy 256 x 16384")
    x, t = to_device(w)
    n = gpu_lib.skl_recommended_splits(t["q1"], t["k1"], t["q2"], t["k2"], False)
    assert n > 1
    ws, n = gpu_lib.skl_forward_splitk(t["q1"], t["k1"], t["q2"], t["k2"], w.scale1, w.scale2, False, n)
    kl, l1, l2 = gpu_lib.skl_reduce(ws, n, w.B, w.H, w.NQ)
    torch.cuda.synchronize()
    got = {"kl": kl.cpu().numpy(), "lse1": l1.cpu().numpy(), "lse2": l2.cpu().numpy()}
    check_rows(w.name, w, got, oracle_forward(w, x))


@pytest.mark.parametrize("algo", ["split", "fused_atomic"])
def test_backward_run_to_run_variation(gpu_lib, algo):
    """The split backward is bitwise deterministic; atomic dQ accumulation
    changes only the rounding order."""
    w = W("rerun", 1, 2, 384, 384, 128, 128, "bf16", True)
    say(f"[backward rerun {algo}]")
    x, t = to_device(w)
    _, (kl, l1, l2) = gpu_forward(gpu_lib, w, t)
    outs = []
    for _ in range(3):
        dq, dk = gpu_lib.skl_backward_student(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, t["g"],
                                              w.scale1, w.scale2, w.causal, algo=algo)
        outs.append((dq.float().clone(), dk.float().clone()))
    torch.cuda.synchronize()
    for dq, dk in outs[1:]:
        assert torch.equal(dk, outs[0][1]), "dK is accumulated on chip: bitwise reproducible"
        if algo == "split":
            assert torch.equal(dq, outs[0][0])
        rel = float((dq - outs[0][0]).norm() / outs[0][0].norm())
        assert rel <= 1e-2 * 1e-2


KEY_SPLIT_CASES = [
    W("ks_bf16_causal_chunk", 1, 2, 100, 3000, 128, 128, "bf16", True, synth.Recipe("corr", noise=0.3)),
    W("ks_bf16_noncausal", 1, 1, 200, 2100, 128, 64, "bf16", False),
    W("ks_f32_causal", 1, 1, 130, 1500, 64, 64, "f32", True),
    W("ks_bf16_causal_square", 1, 1, 700, 700, 64, 128, "bf16", True),
]


@pytest.mark.parametrize("setting", ["student", "teacher"])
@pytest.mark.parametrize("w", KEY_SPLIT_CASES, ids=lambda w: w.name)
def test_backward_dq_key_ranges(gpu_lib, w, setting):
    """Few query tiles: the split backward's dQ kernel cuts the keys into
    ranges whose partials are summed.  Against the oracle, against the
    unsplit dQ (zero-size workspace), and bitwise repeatable."""
    say(f"[backward dQ key ranges {setting}] {w.name}")
    x, t = to_device(w)
    _, (kl, l1, l2) = gpu_forward(gpu_lib, w, t)
    assert gpu_lib.skl_backward_workspace_size(t["q1"], t["k1"], t["q2"], t["k2"], setting == "teacher") > 0

    def run(ws=None):
        if setting == "student":
            return gpu_lib.skl_backward_student(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, t["g"],
                                                w.scale1, w.scale2, w.causal, ws=ws)
        return gpu_lib.skl_backward_teacher(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, kl, t["g"],
                                            w.scale1, w.scale2, w.causal, ws=ws)

    dq, dk = run()
    dq_again, _ = run()
    dq_whole, dk_whole = run(ws=torch.empty(0, dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    rq, rk = oracle_backward(w, x, setting)
    check_grad(f"{w.name} dQ ({setting}, key ranges)", w, grad_to_np(dq), rq)
    check_grad(f"{w.name} dK ({setting})", w, grad_to_np(dk), rk)
    check_grad(f"{w.name} dQ ({setting}, unsplit)", w, grad_to_np(dq_whole), rq)
    assert torch.equal(dq, dq_again), "key-range partials are summed in a fixed order"
    assert torch.equal(dk, dk_whole), "dK does not depend on the dQ key ranges"
    rel = float((dq.float() - dq_whole.float()).norm() / dq_whole.float().norm())
    assert rel <= TOL[w.dtype]["grad"]


def test_split_and_fused_backward_agree(gpu_lib):
    w = W("agree", 2, 2, 300, 300, 128, 64, "bf16", True, synth.Recipe("iid", amp1=2.0))
    say("[backward split vs fused]")
    x, t = to_device(w)
    _, (kl, l1, l2) = gpu_forward(gpu_lib, w, t)
    a = gpu_lib.skl_backward_teacher(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, kl, t["g"], w.scale1,
                                     w.scale2, True, algo="split")
    b = gpu_lib.skl_backward_teacher(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, kl, t["g"], w.scale1,
                                     w.scale2, True, algo="fused_atomic")
    torch.cuda.synchronize()
    for x_, y_ in zip(a, b):
        rel = float((x_.float() - y_.float()).norm() / y_.float().norm())
        assert rel <= 1e-2


def test_errors_raise_before_launch(gpu_lib):
    w = W("err", 1, 1, 64, 64, 128, 128, "bf16", False)
    _, t = to_device(w)
    with pytest.raises(gpu_lib.SklError):
        gpu_lib.skl_forward(t["q1"], t["k1"], t["q2"], t["k2"], 0.0, 0.1, False)
    with pytest.raises(gpu_lib.SklError):
        gpu_lib.skl_forward(t["q1"][..., :96].contiguous(), t["k1"][..., :96].contiguous(),
                            t["q2"], t["k2"], 0.1, 0.1, False)


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_joint_backward_matches_oracle(gpu_lib, w):
    """Both settings in one pass (joint kernels, no workspace): all four
    gradients against the oracle, and against the two separate calls."""
    say(f"[joint backward] {w.name}")
    x, t = to_device(w)
    _, (kl, l1, l2) = gpu_forward(gpu_lib, w, t)
    none = torch.empty(0, dtype=torch.float32, device="cuda")
    dq1, dk1, dq2, dk2 = gpu_lib.skl_backward_joint(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, kl, t["g"],
                                                    w.scale1, w.scale2, w.causal, ws=none)
    again = gpu_lib.skl_backward_joint(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, kl, t["g"],
                                       w.scale1, w.scale2, w.causal, ws=none)
    sq2, sk2 = gpu_lib.skl_backward_student(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, t["g"],
                                            w.scale1, w.scale2, w.causal, ws=none)
    sq1, sk1 = gpu_lib.skl_backward_teacher(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, kl, t["g"],
                                            w.scale1, w.scale2, w.causal, ws=none)
    torch.cuda.synchronize()
    for a, b_ in zip((dq1, dk1, dq2, dk2), again):
        assert torch.equal(a, b_), "joint backward is bitwise deterministic"
    for setting, dq, dk, sq, sk in (("teacher", dq1, dk1, sq1, sk1), ("student", dq2, dk2, sq2, sk2)):
        rq, rk = oracle_backward(w, x, setting)
        check_grad(f"{w.name} joint dQ ({setting})", w, grad_to_np(dq), rq)
        check_grad(f"{w.name} joint dK ({setting})", w, grad_to_np(dk), rk)
        # The split dQ kernel forms sign(g) dS with log2 |g| inside the
        # exponent, the joint kernels multiply by g: the two agree to the
        # rounding of the outputs (bf16: 2^-9 relative per element), or to
        # fp32 noise where the gradient is exactly 0 in real arithmetic (a
        # row with one key), as check_grad allows against the oracle.
        rel = 1e-5 if w.dtype == "f32" else 2e-3
        for a, b_ in ((dq, sq), (dk, sk)):
            den = float(b_.float().norm())
            assert float((a.float() - b_.float()).norm()) <= rel * den + 1e-6


@pytest.mark.parametrize("w", KEY_SPLIT_CASES[:2], ids=lambda w: w.name)
def test_joint_backward_with_key_range_workspace(gpu_lib, w):
    """Few query tiles and the workspace: the joint call runs both settings
    with key-split dQ."""
    say(f"[joint backward, key ranges] {w.name}")
    x, t = to_device(w)
    _, (kl, l1, l2) = gpu_forward(gpu_lib, w, t)
    assert gpu_lib.skl_backward_joint_workspace_size(t["q1"], t["k1"], t["q2"], t["k2"]) > 0
    dq1, dk1, dq2, dk2 = gpu_lib.skl_backward_joint(t["q1"], t["k1"], t["q2"], t["k2"], l1, l2, kl, t["g"],
                                                    w.scale1, w.scale2, w.causal)
    torch.cuda.synchronize()
    for setting, dq, dk in (("teacher", dq1, dk1), ("student", dq2, dk2)):
        rq, rk = oracle_backward(w, x, setting)
        check_grad(f"{w.name} joint dQ ({setting})", w, grad_to_np(dq), rq)
        check_grad(f"{w.name} joint dK ({setting})", w, grad_to_np(dk), rk)


@pytest.mark.parametrize("call", ["student", "teacher", "joint", "fused_atomic"])
def test_backward_without_query_rows_zeroes_key_gradients(gpu_lib, call):
    """N_Q = 0 < N_K: no query sees any key, so every key gradient is exactly
    zero and the call must write it (the outputs are fresh allocations; the
    same-sized blocks are first filled with NaN and handed back to the
    allocator, so memory left unwritten would show)."""
    say(f"[no query rows] {call}")
    B, H, NK, d1, d2 = 2, 3, 77, 128, 64
    g = torch.Generator(device="cpu").manual_seed(5)
    k1 = torch.randn(B, H, NK, d1, generator=g).to("cuda", torch.bfloat16)
    k2 = torch.randn(B, H, NK, d2, generator=g).to("cuda", torch.bfloat16)
    q1 = torch.empty(B, H, 0, d1, dtype=torch.bfloat16, device="cuda")
    q2 = torch.empty(B, H, 0, d2, dtype=torch.bfloat16, device="cuda")
    rows = [torch.empty(B, H, 0, dtype=torch.float32, device="cuda") for _ in range(4)]
    for t in (k1, k2, k1, k2):
        junk = torch.full_like(t, float("nan"))
        del junk
    if call == "student":
        dks = [gpu_lib.skl_backward_student(q1, k1, q2, k2, rows[0], rows[1], rows[3], causal=True)[1]]
    elif call == "teacher":
        dks = [gpu_lib.skl_backward_teacher(q1, k1, q2, k2, *rows, causal=True)[1]]
    elif call == "joint":
        _, dk1, _, dk2 = gpu_lib.skl_backward_joint(q1, k1, q2, k2, *rows, causal=True)
        dks = [dk1, dk2]
    else:
        dks = [gpu_lib.skl_backward_student(q1, k1, q2, k2, rows[0], rows[1], rows[3], algo="fused_atomic")[1],
               gpu_lib.skl_backward_teacher(q1, k1, q2, k2, *rows, algo="fused_atomic")[1]]
    torch.cuda.synchronize()
    for dk in dks:
        assert dk.shape[2] == NK and torch.equal(dk, torch.zeros_like(dk)), f"{call}: key gradient not zero"
