"""Algorithmic work of the attention-KL hot path (pure arithmetic, no GPU).

"Pairs" are the unmasked (query, key) pairs: B*H*N_Q*N_K, or, for bottom-right
causal attention, B*H*sum_i (i + N_K - N_Q + 1).

Per pair the method must do (it cannot skip any of it):
  forward            2*(d1 + d2) MFMA flops (both logits), 2 exponentials
  student backward   2*(d1 + 3*d2) flops (both logits, dK2 and dQ2), 2 exponentials
  teacher backward   2*(3*d1 + d2) flops (both logits, dK1 and dQ1), 1 exponential
The forward must at least read Q1, K1, Q2, K2 once and write KL and two LSE
rows; materialising both distributions instead takes 2*B*H*N_Q*N_K elements.
"""
from __future__ import annotations

from dataclasses import dataclass


def pairs(B: int, H: int, NQ: int, NK: int, causal: bool) -> int:
    if not causal:
        return B * H * NQ * NK
    off = NK - NQ
    return B * H * (NQ * (off + 1) + NQ * (NQ - 1) // 2)


@dataclass(frozen=True)
class Work:
    pairs: int
    fwd_flops: int
    student_flops: int
    teacher_flops: int
    fwd_exps: int
    student_exps: int
    teacher_exps: int
    fwd_bytes: int        # compulsory HBM bytes of the forward
    student_bytes: int    # compulsory HBM bytes of the student backward (no workspace)
    teacher_bytes: int
    materialised_bytes: int  # both N_Q x N_K distributions in the input dtype


def work(B, H, NQ, NK, d1, d2, causal, elem_bytes=2) -> Work:
    p = pairs(B, H, NQ, NK, causal)
    inputs = B * H * (NQ + NK) * (d1 + d2) * elem_bytes
    rowvec = B * H * NQ * 4
    return Work(
        pairs=p,
        fwd_flops=2 * p * (d1 + d2),
        student_flops=2 * p * (d1 + 3 * d2),
        teacher_flops=2 * p * (3 * d1 + d2),
        fwd_exps=2 * p,
        student_exps=2 * p,
        teacher_exps=p,
        fwd_bytes=inputs + 3 * rowvec,
        student_bytes=inputs + 3 * rowvec + B * H * (NQ + NK) * d2 * elem_bytes,
        teacher_bytes=inputs + 4 * rowvec + B * H * (NQ + NK) * d1 * elem_bytes,
        materialised_bytes=materialised_bytes(B, H, NQ, NK, elem_bytes),
    )


def materialised_bytes(B, H, NQ, NK, elem_bytes=2, distributions=2) -> int:
    """Bytes to hold the attention distributions explicitly."""
    return distributions * B * H * NQ * NK * elem_bytes


# MI355X published peaks used as roofline denominators.
PEAK_BF16_DENSE_TFLOPS = 2500.0
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
