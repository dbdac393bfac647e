"""Seeded synthetic inputs for the attention-KL primitive.

This module only draws and rounds inputs: it holds none of the method's
arithmetic, so the float64 oracle and the HIP path can both be fed from it.

Every tensor of one (workload, tensor, batch, head) comes from its own
``numpy`` ``SeedSequence`` stream, so any single head can be regenerated on its
own (the oracle checks sampled heads of the large workloads that way).  Values
are drawn as float32 standard normals, composed in float32 following the
workload's recipe, then rounded to the workload's dtype grid (bf16 by
round-to-nearest-even through torch, or left in float32).  The returned numpy
arrays hold exactly the values the GPU receives.

Workload shapes and recipes follow the StreamKL evaluation settings: a tiny
fp32 case, 4K causal, 16K causal/non-causal, 64K causal with 32 heads, and 128K
causal with an indexer-style d=64 student (StreamKL paper digest page,
"Abstract"; agidaily.cc StreamKL article, "Results" and the long-context claims
there).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np

# Tensor ids of the per-(b, h) streams.
T_Q1, T_K1, T_Q2, T_K2, T_G = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Recipe:
    """How Q1, K1, Q2, K2 are composed from independent N(0,1) draws.

    kind:
      "iid"        Q1, K1, Q2, K2 independent; Q1 *= amp1, Q2 *= amp2.
      "corr"       Q1, K1 ~ N(0,1); Q2 = Q1 + noise*eQ, K2 = K1 + noise*eK
                   (needs d1 == d2); then Q1 *= amp1, Q2 *= amp2.
      "identical"  Q2 = Q1 and K2 = K1 (bitwise), Q1 *= amp1 first.
      "uniform1"   like "iid" but Q1 = 0, so the teacher rows are uniform.

    kramp > 0 then scales key row j of K1 and K2 by 1 + kramp * j / (NK - 1),
    so logits grow along the key axis and later keys overtake every earlier
    row maximum by a wide margin.
    """

    kind: str = "iid"
    noise: float = 0.0
    amp1: float = 1.0
    amp2: float = 1.0
    kramp: float = 0.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    NQ: int
    NK: int
    d1: int
    d2: int
    dtype: str  # "bf16" or "f32"
    causal: bool
    scale1: float
    scale2: float
    recipe: Recipe = Recipe()
    grad: str = "mean"  # "mean": g = 1/(B*H*NQ);  "random": g ~ N(0,1)
    seed: int = 0

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def heads(self) -> int:
        return self.B * self.H


def _isqrt(d: int) -> float:
    return 1.0 / math.sqrt(d)


# The five evaluation workloads.  Sizes follow the settings the StreamKL pages
# discuss (64K context with 32 heads; 128K context; 16K; short contexts).
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_f32_n256_d64", 1, 1, 256, 256, 64, 64, "f32", False,
                 _isqrt(64), _isqrt(64), Recipe("iid"), "mean", seed=101),
        Workload("causal_4k_h8x2_d128_corr03", 2, 8, 4096, 4096, 128, 128, "bf16", True,
                 _isqrt(128), _isqrt(128), Recipe("corr", noise=0.3), "mean", seed=102),
        Workload("n16k_h32_d128_corr05", 1, 32, 16384, 16384, 128, 128, "bf16", True,
                 _isqrt(128), _isqrt(128), Recipe("corr", noise=0.5), "mean", seed=103),
        Workload("causal_64k_h32_d128_q1x4", 1, 32, 65536, 65536, 128, 128, "bf16", True,
                 _isqrt(128), _isqrt(128), Recipe("iid", amp1=4.0), "mean", seed=104),
        Workload("causal_128k_h8_d128_d64", 1, 8, 131072, 131072, 128, 64, "bf16", True,
                 _isqrt(128), _isqrt(64), Recipe("iid"), "mean", seed=105),
        # Long contexts on one GPU (the pages claim up to 512K).
        Workload("causal_256k_h4_d128", 1, 4, 262144, 262144, 128, 128, "bf16", True,
                 _isqrt(128), _isqrt(128), Recipe("corr", noise=0.5), "mean", seed=106),
        Workload("causal_512k_h2_d128", 1, 2, 524288, 524288, 128, 128, "bf16", True,
                 _isqrt(128), _isqrt(128), Recipe("corr", noise=0.5), "mean", seed=107),
        # A 1024-query chunk at the end of a 256K causal sequence (bottom-right
        # aligned): few query tiles, many keys -- the split-K regime.
        Workload("chunk_1k_of_256k_h8_d128", 1, 8, 1024, 262144, 128, 128, "bf16", True,
                 _isqrt(128), _isqrt(128), Recipe("corr", noise=0.3), "mean", seed=108),
    ]
}

WORKLOAD_ORDER = list(WORKLOADS)


def _stream(seed: int, tensor: int, b: int, h: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tensor, b, h]))


def _normal(seed: int, tensor: int, b: int, h: int, n: int, d: int) -> np.ndarray:
    return _stream(seed, tensor, b, h).standard_normal((n, d), dtype=np.float32)


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values onto the dtype grid; returns float32 holding them."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        import torch

        return torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    raise ValueError(f"unknown dtype {dtype!r}")


def head_inputs(w: Workload, b: int, h: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """(Q1, K1, Q2, K2) of one (b, h) as float32 arrays on the dtype grid."""
    r = w.recipe
    s = w.seed
    if r.kind == "corr":
        if w.d1 != w.d2:
            raise ValueError("the correlated recipe needs d1 == d2")
        q1 = _normal(s, T_Q1, b, h, w.NQ, w.d1)
        k1 = _normal(s, T_K1, b, h, w.NK, w.d1)
        q2 = q1 + np.float32(r.noise) * _normal(s, T_Q2, b, h, w.NQ, w.d2)
        k2 = k1 + np.float32(r.noise) * _normal(s, T_K2, b, h, w.NK, w.d2)
    elif r.kind in ("iid", "uniform1"):
        q1 = _normal(s, T_Q1, b, h, w.NQ, w.d1)
        k1 = _normal(s, T_K1, b, h, w.NK, w.d1)
        q2 = _normal(s, T_Q2, b, h, w.NQ, w.d2)
        k2 = _normal(s, T_K2, b, h, w.NK, w.d2)
        if r.kind == "uniform1":
            q1 = np.zeros_like(q1)
    elif r.kind == "identical":
        if w.d1 != w.d2:
            raise ValueError("the identical recipe needs d1 == d2")
        q1 = _normal(s, T_Q1, b, h, w.NQ, w.d1)
        k1 = _normal(s, T_K1, b, h, w.NK, w.d1)
        q2, k2 = q1, k1
    else:
        raise ValueError(f"unknown recipe {r.kind!r}")
    if r.amp1 != 1.0:
        q1 = q1 * np.float32(r.amp1)
    if r.amp2 != 1.0 and r.kind != "identical":
        q2 = q2 * np.float32(r.amp2)
    if r.kramp:
        ramp = (1.0 + r.kramp * np.arange(w.NK) / max(w.NK - 1, 1)).astype(np.float32)[:, None]
        k1 = k1 * ramp
        k2 = k2 * ramp if r.kind != "identical" else k1
    if r.kind == "identical":
        q1 = round_to_dtype(q1, w.dtype)
        k1 = round_to_dtype(k1, w.dtype)
        return q1, k1, q1.copy(), k1.copy()
    return tuple(round_to_dtype(x, w.dtype) for x in (q1, k1, q2, k2))  # type: ignore[return-value]


def head_grad(w: Workload, b: int, h: int) -> np.ndarray:
    """Upstream gradient dL/dKL for the rows of one (b, h), float32 [NQ]."""
    if w.grad == "mean":
        return np.full(w.NQ, 1.0 / (w.B * w.H * w.NQ), dtype=np.float32)
    if w.grad == "random":
        return _stream(w.seed, T_G, b, h).standard_normal(w.NQ, dtype=np.float32)
    raise ValueError(f"unknown grad recipe {w.grad!r}")


def all_inputs(w: Workload) -> Dict[str, np.ndarray]:
    """Every head stacked as [B, H, N, d] float32 (small workloads only)."""
    out = {k: [] for k in ("q1", "k1", "q2", "k2", "g")}
    for b in range(w.B):
        for h in range(w.H):
            q1, k1, q2, k2 = head_inputs(w, b, h)
            for k, v in zip(("q1", "k1", "q2", "k2"), (q1, k1, q2, k2)):
                out[k].append(v)
            out["g"].append(head_grad(w, b, h))
    res = {}
    for k, v in out.items():
        a = np.stack(v)
        res[k] = a.reshape((w.B, w.H) + a.shape[1:])
    return res


def device_inputs(w: Workload, device: str = "cuda", layout: str = "bhnd",
                  with_grad: bool = True, heads: Optional[int] = None):
    """Torch tensors of the workload on ``device``, built one head at a time.

    layout "bhnd" gives contiguous [B, H, N, d]; "bnhd" gives a [B, H, N, d]
    view of contiguous [B, N, H, d] storage.  Returns dict with q1, k1, q2, k2
    (bf16 or fp32) and g (fp32 [B, H, NQ]).
    """
    import torch

    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def alloc(n, d):
        if layout == "bhnd":
            return torch.empty((w.B, w.H, n, d), dtype=tdt, device=device)
        if layout == "bnhd":
            return torch.empty((w.B, n, w.H, d), dtype=tdt, device=device).transpose(1, 2)
        raise ValueError(layout)

    q1, k1 = alloc(w.NQ, w.d1), alloc(w.NK, w.d1)
    q2, k2 = alloc(w.NQ, w.d2), alloc(w.NK, w.d2)
    g = torch.empty((w.B, w.H, w.NQ), dtype=torch.float32, device=device)
    for b in range(w.B):
        for h in range(w.H):
            hq1, hk1, hq2, hk2 = head_inputs(w, b, h)
            for dst, src in ((q1, hq1), (k1, hk1), (q2, hq2), (k2, hk2)):
                dst[b, h].copy_(torch.from_numpy(src).to(tdt))
            if with_grad:
                g[b, h].copy_(torch.from_numpy(head_grad(w, b, h)))
    return {"q1": q1, "k1": k1, "q2": q2, "k2": k2, "g": g}
