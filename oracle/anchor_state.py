"""Anchor-state reuse: the anchor pass's attention state and the sparse pass that resumes
from it (oracle, CPU, fp64).

TEST INFRASTRUCTURE -- see the package docstring.

Sources (AnchorAttention: Difference-Aware Sparse Attention with Stripe Granularity,
arXiv 2505.23520, review page):
* "What carries the argument": the kernel caches what the anchor computation produced and
  the sparse computation starts from it;
* referee major comment 1: the anchor kernel keeps, per query row, the running row max (the
  M buffer) and the p.V accumulator (Acc) of an online softmax;
* referee minor comment 2: the sparse loop starts past the initial key block, which the
  anchor computation has already covered.

Readings (the pages name the reuse but do not spell it out):
* the anchor region of row r is the token set of Eq. (1)'s max,
  A(r) = {j <= r : j < sink or j >= r - local + 1};
* the anchor pass keeps, per (batch, query head, row), the softmax attention over A(r) as a
  normalised partial output O_A(r) and its log-sum-exp LSE_A(r) -- the same information as
  (M, Acc, and the row sum): O_A = Acc / l, LSE_A = M + ln l;
* the sparse pass covers the listed causal tokens outside A(r) (O_B, LSE_B) and merges with
  LSE = ln(e^LSE_A + e^LSE_B), O = e^(LSE_A - LSE) O_A + e^(LSE_B - LSE) O_B;
* every list of the estimate holds the forced blocks, which contain A(r) for every row r of
  the query block, so the merged result is the attention over the list itself.
"""
from __future__ import annotations

import numpy as np

from .estimate import _f64, softmax_scale, query_block_rows


def anchor_region(r: int, sink: int, local: int) -> np.ndarray:
    """A(r) as ascending token ids."""
    lo = max(0, r - local + 1)
    return np.union1d(np.arange(min(sink, r + 1)), np.arange(lo, r + 1)).astype(np.int64)


def _softmax_rows(z: np.ndarray, vf: np.ndarray):
    """Per row of z (scores, -inf = excluded): O = softmax(z) v and LSE; rows with no
    finite score (an empty token set included) give O = 0 and LSE = -inf."""
    if z.shape[1] == 0:
        return np.zeros((z.shape[0], vf.shape[1])), np.full(z.shape[0], -np.inf)
    m = z.max(axis=1, keepdims=True)
    ok = np.isfinite(m)
    ms = np.where(ok, m, 0.0)
    p = np.where(np.isfinite(z), np.exp(z - ms), 0.0)
    s = p.sum(axis=1, keepdims=True)
    o = np.where(ok, (p / np.where(ok, s, 1.0)) @ vf, 0.0)
    lse = np.where(ok, ms + np.log(np.where(ok, s, 1.0)), -np.inf)[:, 0]
    return o, lse


def anchor_state_rows(q, k, v, *, block_q: int, sink: int, local: int, rows,
                      scale: float | None = None, kv_of_q=None) -> dict:
    """State of the anchor pass for the query blocks ``rows`` = iterable of (b, h, i).

    Returns {(b, h, i): (O_A [rows, d] float64, LSE_A [rows] float64)}."""
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    c = float(softmax_scale(D, scale))
    if kv_of_q is None:
        kv_of_q = np.arange(Hq) // (Hq // Hkv)
    out = {}
    for (b, h, i) in rows:
        g = int(kv_of_q[h])
        r0, r1 = query_block_rows(i, N, block_q)
        lo = max(0, r0 - local + 1)
        toks = np.union1d(np.arange(min(sink, r1)), np.arange(lo, r1)).astype(np.int64)
        kf = _f64(k[b, toks, g, :])
        vf = _f64(v[b, toks, g, :])
        qb = _f64(q[b, r0:r1, h, :])
        z = c * (qb @ kf.T)
        rr = np.arange(r0, r1)[:, None]
        j = toks[None, :]
        allowed = (j <= rr) & ((j < sink) | (j >= rr - local + 1))
        out[(b, h, i)] = _softmax_rows(np.where(allowed, z, -np.inf), vf)
    return out


def merge_partials(o_a, lse_a, o_b, lse_b):
    """Attention over the union of two disjoint token sets from the attention over each
    (normalised outputs and log-sum-exps; an empty set has LSE = -inf)."""
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    lse = np.logaddexp(lse_a, lse_b)
    fin = np.isfinite(lse)
    safe = np.where(fin, lse, 0.0)
    wa = np.where(np.isfinite(lse_a) & fin, np.exp(lse_a - safe), 0.0)
    wb = np.where(np.isfinite(lse_b) & fin, np.exp(lse_b - safe), 0.0)
    o = wa[:, None] * np.asarray(o_a, dtype=np.float64) + wb[:, None] * np.asarray(o_b, dtype=np.float64)
    return o, lse


def resume_rows(q, k, v, lists, state, *, block_q: int, block_k: int, sink: int, local: int,
                rows, scale: float | None = None, kv_of_q=None, granularity: str = "block") -> dict:
    """The sparse pass that resumes from the anchor state: attention over the tokens of the
    list of (b, g, i) (key blocks, or key columns with granularity "stripe") that are causal
    for row r and outside A(r), merged with ``state[(b, h, i)]``.  Returns
    {(b, h, i): (O [rows, d], LSE [rows])}."""
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    c = float(softmax_scale(D, scale))
    if kv_of_q is None:
        kv_of_q = np.arange(Hq) // (Hq // Hkv)
    out = {}
    for (b, h, i) in rows:
        g = int(kv_of_q[h])
        r0, r1 = query_block_rows(i, N, block_q)
        kept = np.asarray(lists[(b, g, i)], dtype=np.int64)
        if granularity == "stripe":
            toks = kept[kept < N]
        else:
            toks = (kept[:, None] * block_k + np.arange(block_k)[None, :]).reshape(-1)
            toks = toks[toks < N]
        kf = _f64(k[b, toks, g, :])
        vf = _f64(v[b, toks, g, :])
        qb = _f64(q[b, r0:r1, h, :])
        z = c * (qb @ kf.T)
        rr = np.arange(r0, r1)[:, None]
        j = toks[None, :]
        in_anchor = (j < sink) | (j >= rr - local + 1)
        o_b, lse_b = _softmax_rows(np.where((j <= rr) & ~in_anchor, z, -np.inf), vf)
        o_a, lse_a = state[(b, h, i)]
        out[(b, h, i)] = merge_partials(o_a, lse_a, o_b, lse_b)
    return out
