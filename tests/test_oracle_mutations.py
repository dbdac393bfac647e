"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch each one.  A pin set that lets a mutant through is too weak."""
import numpy as np
import pytest

import oracle.streamkl_oracle as orc
from tests import test_oracle_pins as pins

_orig_row_block = orc._row_block
_orig_dS = orc._dS


def _rb_kl_sign(*a):
    r = _orig_row_block(*a)
    r["kl"] = -r["kl"]
    return r


def _rb_drop_scale2(q1, k1, q2, k2, s1, s2, causal, rows):
    return _orig_row_block(q1, k1, q2, k2, s1, 1.0, causal, rows)


def _rb_mask_off_by_one(q1, k1, q2, k2, s1, s2, causal, rows):
    r = _orig_row_block(q1, k1, q2, k2, s1, s2, False, rows)
    if causal:
        nq, nk = q1.shape[0], k1.shape[0]
        allow = np.arange(nk)[None, :] < (np.asarray(rows)[:, None] + nk - nq)
        allow[:, 0] = True
        for k in ("s1", "s2"):
            r[k] = np.where(allow, r[k], -np.inf)
        r.update(_recompute(r, allow))
    return r


def _recompute(r, allow):
    out = {"allow": allow}
    out["lse1"] = orc.row_logsumexp(r["s1"], allow)
    out["lse2"] = orc.row_logsumexp(r["s2"], allow)
    out["logp1"] = np.where(allow, r["s1"] - out["lse1"][:, None], 0.0)
    out["logp2"] = np.where(allow, r["s2"] - out["lse2"][:, None], 0.0)
    out["p1"] = np.where(allow, np.exp(out["logp1"]), 0.0)
    out["p2"] = np.where(allow, np.exp(out["logp2"]), 0.0)
    out["kl"] = np.where(allow, out["p1"] * (out["logp1"] - out["logp2"]), 0.0).sum(1)
    return out


def _rb_p2_from_s1(*a):
    r = _orig_row_block(*a)
    r["logp2"] = r["s1"] - r["lse2"][:, None]
    r["kl"] = np.where(r["allow"], r["p1"] * (r["logp1"] - r["logp2"]), 0.0).sum(1)
    return r


def _dS_student_sign(r, g, setting):
    ds = _orig_dS(r, g, setting)
    return -ds if setting == "student" else ds


def _dS_teacher_no_kl(r, g, setting):
    if setting != "teacher":
        return _orig_dS(r, g, setting)
    g = np.asarray(g, dtype=np.float64)[:, None]
    return np.where(r["allow"], g * r["p1"] * (r["logp1"] - r["logp2"]), 0.0)


def _dS_teacher_p2(r, g, setting):
    if setting != "teacher":
        return _orig_dS(r, g, setting)
    g = np.asarray(g, dtype=np.float64)[:, None]
    ratio = np.where(r["allow"], r["logp1"] - r["logp2"], 0.0)
    return np.where(r["allow"], g * r["p2"] * (ratio - r["kl"][:, None]), 0.0)


def _dS_transposed_rows(r, g, setting):
    ds = _orig_dS(r, g, setting)
    return ds[::-1].copy()


def _run_forward_pins():
    pins.test_kl_is_nonnegative(1, True)
    pins.test_uniform_teacher_closed_form(True, 9, 25)
    pins.test_two_key_bernoulli_closed_form()
    for causal in (False, True):
        pins.test_forward_matches_scalar_brute_force((7, 7, 4, 3), causal)
        pins.test_forward_matches_scalar_brute_force((5, 11, 4, 4), causal)


def _run_backward_pins():
    for setting in ("student", "teacher"):
        for causal in (False, True):
            pins.test_gradients_match_finite_differences(setting, causal, (5, 5, 4, 2))
            pins.test_key_gradients_sum_to_zero(setting, causal)


@pytest.mark.parametrize("mutant", [_rb_kl_sign, _rb_drop_scale2, _rb_mask_off_by_one, _rb_p2_from_s1])
def test_forward_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(orc, "_row_block", mutant)
    with pytest.raises(AssertionError):
        _run_forward_pins()


@pytest.mark.parametrize("mutant", [_dS_student_sign, _dS_teacher_no_kl, _dS_teacher_p2, _dS_transposed_rows])
def test_backward_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(orc, "_dS", mutant)
    with pytest.raises(AssertionError):
        _run_backward_pins()


def test_unmutated_oracle_passes_the_same_pins():
    _run_forward_pins()
    _run_backward_pins()


# ------------------------------------------ mutants of the batched wrappers ----

import oracle  # noqa: E402  (the package re-exports forward/backward by name)

_orig_forward = orc.forward
_orig_backward = orc.backward


def _fwd_swapped_scales(q1, k1, q2, k2, scale1, scale2, causal):
    return _orig_forward(q1, k1, q2, k2, scale2, scale1, causal)


def _fwd_wrong_head(q1, k1, q2, k2, scale1, scale2, causal):
    """K2 taken from the next head (a plausible indexing slip in the loop)."""
    out = _orig_forward(q1, k1, q2, k2, scale1, scale2, causal)
    H = q1.shape[1]
    for b in range(q1.shape[0]):
        for h in range(H):
            r = orc.head_forward(q1[b, h], k1[b, h], q2[b, h], k2[b, (h + 1) % H], scale1, scale2, causal)
            for k in out:
                out[k][b, h] = r[k]
    return out


def _bwd_wrong_head_g(q1, k1, q2, k2, scale1, scale2, causal, g, setting):
    return _orig_backward(q1, k1, q2, k2, scale1, scale2, causal, g[:, ::-1].copy(), setting)


def _bwd_swapped_scales(q1, k1, q2, k2, scale1, scale2, causal, g, setting):
    return _orig_backward(q1, k1, q2, k2, scale2, scale1, causal, g, setting)


def _bwd_wrong_head_out(q1, k1, q2, k2, scale1, scale2, causal, g, setting):
    """dK of head h stored into head h + 1."""
    dq, dk = _orig_backward(q1, k1, q2, k2, scale1, scale2, causal, g, setting)
    return dq, np.roll(dk, 1, axis=1)


def _run_batched_forward_pins():
    for causal in (False, True):
        pins.test_batched_forward_matches_brute_force_per_head(causal)


def _run_batched_backward_pins():
    for setting in ("student", "teacher"):
        for causal in (False, True):
            pins.test_batched_backward_matches_finite_differences(setting, causal)


@pytest.mark.parametrize("mutant", [_fwd_swapped_scales, _fwd_wrong_head])
def test_batched_forward_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(orc, "forward", mutant)
    monkeypatch.setattr(oracle, "forward", mutant)
    with pytest.raises(AssertionError):
        _run_batched_forward_pins()


@pytest.mark.parametrize("mutant", [_bwd_wrong_head_g, _bwd_swapped_scales, _bwd_wrong_head_out])
def test_batched_backward_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(orc, "backward", mutant)
    monkeypatch.setattr(oracle, "backward", mutant)
    with pytest.raises(AssertionError):
        _run_batched_backward_pins()


def test_unmutated_batched_wrappers_pass_the_same_pins():
    _run_batched_forward_pins()
    _run_batched_backward_pins()
