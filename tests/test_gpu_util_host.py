"""Host-side checks of the GPU parity helpers (no GPU needed): the gradient
comparison must reject a single wrong row that a tensor-wide relative L2
bound alone lets through, and accept rounding-sized noise."""
import numpy as np
import pytest

import oracle
from attention_kl_divergence_skl_amd import synth
from tests.gpu_util import TOL, check_grad, rel_l2, worst_row_error


def _reference():
    w = synth.Workload("t", 1, 2, 300, 300, 16, 16, "bf16", True, 0.25, 0.25,
                       synth.Recipe("corr", noise=0.3), "random", seed=3)
    x = synth.all_inputs(w)
    dq, dk = oracle.backward(x["q1"], x["k1"], x["q2"], x["k2"], w.scale1, w.scale2, True, x["g"], "student")
    return w, dq, dk


def test_single_bad_row_is_caught():
    w, dq, _ = _reference()
    bad = dq.copy()
    row = 297  # in the ragged tail of the last 128-row tile
    bad[0, 1, row] *= 1.10
    # The tensor-wide relative L2 stays inside the tolerance...
    assert rel_l2(bad, dq) <= TOL["bf16"]["grad"]
    # ...the per-row bound does not.
    e, i = worst_row_error(bad[0, 1], dq[0, 1])
    assert i == row and e > 0.05
    with pytest.raises(AssertionError):
        check_grad("planted row", w, bad, dq)


def test_rounding_noise_passes():
    w, dq, dk = _reference()
    rng = np.random.default_rng(0)
    for ref in (dq, dk):
        noisy = ref * (1 + 2.0 ** -8 * rng.standard_normal(ref.shape))
        check_grad("bf16-sized noise", w, noisy, ref)
