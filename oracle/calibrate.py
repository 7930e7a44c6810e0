"""Per-head threshold calibration (TEST INFRASTRUCTURE; see the package header).

SALE (arXiv 2505.24179), "Assumptions & free parameters": the per-head threshold tau is
calibrated -- it starts at 0.008 and is halved until the L1 output error
Err(tau) = ||O - O~||_1 / N against full attention meets a user-chosen bound.  The
relative-score test keeps a block when its estimated weight is at least tau times the
anchor's, i.e. anchor - score <= -ln tau: theta = -ln tau in the logit units of
AnchorAttention Eq. (2).

Readings where the page is silent: Err is computed per query head, summing |O - O~| over the
batch, the rows and the head dimensions and dividing by the number of rows (batch * seq);
O is attention with every causal block kept; all heads are evaluated together every round
and every head not yet below the bound halves its tau (the lists are unions over the query
heads of a KV head, so heads are coupled); a head stops halving after ``max_halvings``.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import attention_all
from .estimate import estimate_all
from .estimate_sale import estimate_all_sale


def full_lists(n: int, b: int, hkv: int, block_q: int, block_k: int) -> dict:
    """Every causal key block of every query block: the lists of full (dense) attention."""
    nqb = -(-n // block_q)
    out = {}
    for bb in range(b):
        for g in range(hkv):
            for i in range(nqb):
                e = min(n, (i + 1) * block_q) - 1
                out[(bb, g, i)] = np.arange(e // block_k + 1, dtype=np.int64)
    return out


def head_l1_error(o_ref: np.ndarray, o: np.ndarray) -> np.ndarray:
    """Err_h = sum over batch, rows and dims of |o_ref - o| for head h, / (batch * rows).
    o_ref, o: [B, N, Hq, d]."""
    B, N = o_ref.shape[:2]
    return np.abs(o_ref - o).sum(axis=(0, 1, 3)) / float(B * N)


def calibrate_theta(q, k, v, *, tau0: float = 0.008, err_bound: float = 0.4,
                    max_halvings: int = 16, block_q: int, block_k: int, sink: int, local: int,
                    scale=None, estimator: str = "pooled", kv_of_q=None) -> dict:
    """Returns dict(theta [Hq] float32, err [Hq] float64, halvings [Hq] int, history: list of
    (theta, err) per round).  estimator "relative" calibrates SALE's own element-wise
    estimate (``estimate_sale``) instead of the pooled one.  kv_of_q: the KV head of each
    query head (default h // (Hq / Hkv)), passed to the estimate and the attention."""
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    kw = dict(block_q=block_q, block_k=block_k, kv_of_q=kv_of_q)
    o_ref, _ = attention_all(q, k, v, full_lists(N, B, Hkv, block_q, block_k), scale=scale, **kw)
    theta0 = -math.log(tau0)
    halv = np.zeros(Hq, dtype=np.int64)
    history = []
    while True:
        theta = np.array([theta0 + int(kh) * math.log(2.0) for kh in halv], dtype=np.float32)
        if estimator == "relative":
            est = estimate_all_sale(q, k, theta, sink=sink, local=local, scale=scale,
                                    keep_margins=False, **kw)
        else:
            est = estimate_all(q, k, theta, sink=sink, local=local, granularity="block",
                               scale=scale, keep_margins=False, **kw)
        o, _ = attention_all(q, k, v, {key: r["kept"] for key, r in est.items()}, scale=scale, **kw)
        err = head_l1_error(o_ref, o)
        history.append((theta.copy(), err.copy()))
        grow = ~(err < err_bound) & (halv < max_halvings)
        if not grow.any():
            return dict(theta=theta, err=err, halvings=halv.copy(), history=history)
        halv[grow] += 1
