"""Float64 CPU oracle for the fused attention-KL primitive (StreamKL).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` use it.  It shares no code with the HIP library.

What it computes (per batch b, head h, query row i):

* logits  S1 = scale1 * Q1 K1^T,  S2 = scale2 * Q2 K2^T, over the keys row i may
  attend to (all keys, or j <= i + N_K - N_Q when causal);
* P_k = softmax(S_k) over those keys, LSE_k = log sum_j exp(S_k[j]);
* KL_i = sum_j P1[j] * (log P1[j] - log P2[j])  -- the row-wise attention KL
  that attention distillation minimises (agidaily.cc StreamKL article, section
  "Online formula" 在线公式; StreamKL paper digest, "Abstract").

Backward, for an upstream gradient g_i = dLoss/dKL_i, in the two settings the
article's backward section (反向：基于重计算的 Tile-by-Tile 梯度) names:

* optimise P2 (student, P1 fixed): dS2 = g_i (P2 - P1);
  dQ2 = scale2 * dS2 K2,  dK2 = scale2 * dS2^T Q2.
* optimise P1 (teacher, P2 fixed): r_j = log P1[j] - log P2[j] taken from the
  logits (S1 - LSE1) - (S2 - LSE2), never as the log of a probability;
  dS1 = g_i P1 (r - KL_i);  dQ1 = scale1 * dS1 K1,  dK1 = scale1 * dS1^T Q1.
  (d KL / d S1[j] = P1[j] (r_j - sum_k P1[k] r_k) because sum_k P1[k] = 1.)

The rows are materialised (one block of query rows at a time); matmul, exp and
log are numpy's float64 routines.  Readings where the pages are silent:
natural logarithms (KL and LSE in nats); masked keys are outside both supports;
causal alignment is bottom-right (row i sees keys j <= i + N_K - N_Q, N_Q <= N_K);
no clamping of KL.

``online_forward`` is separate on purpose: it follows the pages' streaming
algorithm (running maxima m1, m2, sums l1, l2 and acc = sum e^(S1-m1)(S1-S2),
rescaled per key tile, finished as KL = acc/l1 + LSE2 - LSE1, article section
"Online formula"), optionally split along the keys with partial statistics
merged afterwards (article section "GPU kernel optimisations", split-K).  The
tests pin it to the definition above.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence, Tuple

import numpy as np

ROW_BLOCK = 256


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def allowed_keys(rows: np.ndarray, nq: int, nk: int, causal: bool) -> np.ndarray:
    """Boolean [len(rows), nk]: may query row i attend to key j."""
    rows = np.asarray(rows, dtype=np.int64)
    if not causal:
        return np.ones((rows.size, nk), dtype=bool)
    if nq > nk:
        raise ValueError("causal attention needs N_Q <= N_K (bottom-right alignment)")
    off = nk - nq
    return np.arange(nk, dtype=np.int64)[None, :] <= (rows[:, None] + off)


def row_logsumexp(s: np.ndarray, allow: np.ndarray) -> np.ndarray:
    """log sum_j exp(s[i, j]) over the allowed j of each row (max-shifted)."""
    sm = np.where(allow, s, -np.inf)
    m = sm.max(axis=1)
    return m + np.log(np.exp(sm - m[:, None]).sum(axis=1))


def _row_block(q1, k1, q2, k2, scale1, scale2, causal, rows):
    """Everything the definition needs for a block of query rows of one head."""
    nq, nk = q1.shape[0], k1.shape[0]
    allow = allowed_keys(rows, nq, nk, causal)
    s1 = scale1 * (_f64(q1)[rows] @ _f64(k1).T)
    s2 = scale2 * (_f64(q2)[rows] @ _f64(k2).T)
    lse1 = row_logsumexp(s1, allow)
    lse2 = row_logsumexp(s2, allow)
    logp1 = s1 - lse1[:, None]
    logp2 = s2 - lse2[:, None]
    p1 = np.where(allow, np.exp(np.where(allow, logp1, 0.0)), 0.0)
    p2 = np.where(allow, np.exp(np.where(allow, logp2, 0.0)), 0.0)
    kl = np.where(allow, p1 * (logp1 - logp2), 0.0).sum(axis=1)
    return dict(allow=allow, s1=s1, s2=s2, lse1=lse1, lse2=lse2,
                logp1=logp1, logp2=logp2, p1=p1, p2=p2, kl=kl)


def _blocks(rows: np.ndarray):
    for a in range(0, rows.size, ROW_BLOCK):
        yield rows[a:a + ROW_BLOCK]


def head_forward(q1, k1, q2, k2, scale1: float, scale2: float, causal: bool,
                 rows: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Per-row KL, LSE1, LSE2 of one head (all rows, or the given ones)."""
    nq = q1.shape[0]
    rows = np.arange(nq) if rows is None else np.asarray(rows, dtype=np.int64)
    out = {k: np.empty(rows.size) for k in ("kl", "lse1", "lse2")}
    pos = 0
    for blk in _blocks(rows):
        r = _row_block(q1, k1, q2, k2, scale1, scale2, causal, blk)
        for k in out:
            out[k][pos:pos + blk.size] = r[k]
        pos += blk.size
    return out


def _dS(r, g_rows: np.ndarray, setting: str) -> np.ndarray:
    g = _f64(g_rows)[:, None]
    if setting == "student":
        return np.where(r["allow"], g * (r["p2"] - r["p1"]), 0.0)
    if setting == "teacher":
        ratio = np.where(r["allow"], r["logp1"] - r["logp2"], 0.0)
        return np.where(r["allow"], g * r["p1"] * (ratio - r["kl"][:, None]), 0.0)
    raise ValueError(f"unknown gradient setting {setting!r}")


def head_backward(q1, k1, q2, k2, scale1: float, scale2: float, causal: bool,
                  g, setting: str) -> Tuple[np.ndarray, np.ndarray]:
    """(dQ, dK) of the optimised side of one head: (dQ2, dK2) for "student",
    (dQ1, dK1) for "teacher"."""
    nq = q1.shape[0]
    qg, kg, sc = (q2, k2, scale2) if setting == "student" else (q1, k1, scale1)
    dq = np.zeros(qg.shape, dtype=np.float64)
    dk = np.zeros(kg.shape, dtype=np.float64)
    for blk in _blocks(np.arange(nq)):
        r = _row_block(q1, k1, q2, k2, scale1, scale2, causal, blk)
        ds = _dS(r, _f64(g)[blk], setting)
        dq[blk] = sc * (ds @ _f64(kg))
        dk += sc * (ds.T @ _f64(qg)[blk])
    return dq, dk


def head_dq_rows(q1, k1, q2, k2, scale1, scale2, causal, g, setting: str,
                 rows: Sequence[int]) -> np.ndarray:
    """dQ of the optimised side for the given query rows only (exact per row)."""
    rows = np.asarray(rows, dtype=np.int64)
    kg, sc = (k2, scale2) if setting == "student" else (k1, scale1)
    out = np.empty((rows.size, kg.shape[1]))
    pos = 0
    for blk in _blocks(rows):
        r = _row_block(q1, k1, q2, k2, scale1, scale2, causal, blk)
        out[pos:pos + blk.size] = sc * (_dS(r, _f64(g)[blk], setting) @ _f64(kg))
        pos += blk.size
    return out


def head_dk_cols(q1, k1, q2, k2, scale1, scale2, causal, g, setting: str,
                 cols: Sequence[int]) -> np.ndarray:
    """dK of the optimised side for the given key columns.  Every query row that
    may attend to one of them is materialised (for causal attention and columns
    near the end of the sequence these are few)."""
    cols = np.asarray(cols, dtype=np.int64)
    nq, nk = q1.shape[0], k1.shape[0]
    qg, sc = (q2, scale2) if setting == "student" else (q1, scale1)
    first = max(0, int(cols.min()) - (nk - nq)) if causal else 0
    out = np.zeros((cols.size, qg.shape[1]))
    for blk in _blocks(np.arange(first, nq)):
        r = _row_block(q1, k1, q2, k2, scale1, scale2, causal, blk)
        ds = _dS(r, _f64(g)[blk], setting)[:, cols]
        out += sc * (ds.T @ _f64(qg)[blk])
    return out


# ---------------------------------------------------------------- batched ----

def forward(q1, k1, q2, k2, scale1, scale2, causal) -> Dict[str, np.ndarray]:
    """[B, H, N, d] inputs -> kl, lse1, lse2 as [B, H, N_Q] float64."""
    B, H, nq = q1.shape[0], q1.shape[1], q1.shape[2]
    out = {k: np.empty((B, H, nq)) for k in ("kl", "lse1", "lse2")}
    for b in range(B):
        for h in range(H):
            r = head_forward(q1[b, h], k1[b, h], q2[b, h], k2[b, h], scale1, scale2, causal)
            for k in out:
                out[k][b, h] = r[k]
    return out


def backward(q1, k1, q2, k2, scale1, scale2, causal, g, setting: str):
    """[B, H, N, d] inputs, g [B, H, N_Q] -> (dQ, dK) float64 of the optimised side."""
    B, H = q1.shape[0], q1.shape[1]
    qg, kg = (q2, k2) if setting == "student" else (q1, k1)
    dq = np.empty(qg.shape)
    dk = np.empty(kg.shape)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h] = head_backward(q1[b, h], k1[b, h], q2[b, h], k2[b, h],
                                               scale1, scale2, causal, g[b, h], setting)
    return dq, dk


# ------------------------------------------- the pages' online algorithm ----

def online_partials(q1, k1, q2, k2, scale1, scale2, causal, block_k: int,
                    key_lo: int = 0, key_hi: Optional[int] = None):
    """Running statistics of one head over keys [key_lo, key_hi), streamed in
    key tiles of ``block_k`` (article section "Forward: single-pass streaming
    kernel" 前向：单遍流式 Kernel).  Returns per-row (m1, l1, m2, l2, acc) in
    natural-log units; acc is relative to m1."""
    nq, nk = q1.shape[0], k1.shape[0]
    key_hi = nk if key_hi is None else key_hi
    rows = np.arange(nq)
    m1 = np.full(nq, -np.inf)
    m2 = np.full(nq, -np.inf)
    l1 = np.zeros(nq)
    l2 = np.zeros(nq)
    acc = np.zeros(nq)
    Q1, Q2 = _f64(q1), _f64(q2)
    for j0 in range(key_lo, key_hi, block_k):
        j1 = min(j0 + block_k, key_hi)
        allow = allowed_keys(rows, nq, nk, causal)[:, j0:j1]
        s1 = np.where(allow, scale1 * (Q1 @ _f64(k1)[j0:j1].T), -np.inf)
        s2 = np.where(allow, scale2 * (Q2 @ _f64(k2)[j0:j1].T), -np.inf)
        m1n = np.maximum(m1, s1.max(axis=1))
        m2n = np.maximum(m2, s2.max(axis=1))
        # Correction factors; a row that has seen no key yet keeps l = acc = 0.
        fin1, fin2 = np.isfinite(m1n), np.isfinite(m2n)
        a1 = np.where(fin1, np.exp(np.where(fin1, m1, 0.0) - np.where(fin1, m1n, 0.0)), 1.0)
        a2 = np.where(fin2, np.exp(np.where(fin2, m2, 0.0) - np.where(fin2, m2n, 0.0)), 1.0)
        base1 = np.where(np.isfinite(m1n), m1n, 0.0)[:, None]
        base2 = np.where(np.isfinite(m2n), m2n, 0.0)[:, None]
        e1 = np.where(allow, np.exp(np.where(allow, s1, 0.0) - base1), 0.0)
        e2 = np.where(allow, np.exp(np.where(allow, s2, 0.0) - base2), 0.0)
        diff = np.where(allow, np.where(allow, s1, 0.0) - np.where(allow, s2, 0.0), 0.0)
        l1 = a1 * l1 + e1.sum(axis=1)
        l2 = a2 * l2 + e2.sum(axis=1)
        acc = a1 * acc + (e1 * diff).sum(axis=1)
        m1, m2 = m1n, m2n
    return m1, l1, m2, l2, acc


def merge_partials(parts):
    """Merge per-split (m1, l1, m2, l2, acc) of the same rows into one state."""
    m1 = np.max([p[0] for p in parts], axis=0)
    m2 = np.max([p[2] for p in parts], axis=0)
    l1 = np.zeros_like(m1)
    l2 = np.zeros_like(m1)
    acc = np.zeros_like(m1)
    for pm1, pl1, pm2, pl2, pacc in parts:
        w1 = np.where(np.isfinite(pm1), np.exp(np.where(np.isfinite(pm1), pm1 - m1, 0.0)), 0.0)
        w2 = np.where(np.isfinite(pm2), np.exp(np.where(np.isfinite(pm2), pm2 - m2, 0.0)), 0.0)
        l1 = l1 + w1 * pl1
        acc = acc + w1 * pacc
        l2 = l2 + w2 * pl2
    return m1, l1, m2, l2, acc


def finish(m1, l1, m2, l2, acc) -> Dict[str, np.ndarray]:
    """KL = acc/l1 + LSE2 - LSE1 with LSE_k = m_k + log l_k (article section
    "Online formula")."""
    lse1 = m1 + np.log(l1)
    lse2 = m2 + np.log(l2)
    return {"kl": acc / l1 + lse2 - lse1, "lse1": lse1, "lse2": lse2}


def online_forward(q1, k1, q2, k2, scale1, scale2, causal, block_k: int = 64,
                   splits: int = 1) -> Dict[str, np.ndarray]:
    """The online formula, streamed over key tiles, optionally split along the
    keys into ``splits`` contiguous ranges whose partials are merged."""
    nk = k1.shape[0]
    chunk = -(-nk // splits)
    parts = [online_partials(q1, k1, q2, k2, scale1, scale2, causal, block_k,
                             s * chunk, min(nk, (s + 1) * chunk)) for s in range(splits)]
    return finish(*merge_partials(parts))
