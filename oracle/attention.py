"""Masked softmax attention under given kept lists (oracle, CPU, fp64).

TEST INFRASTRUCTURE -- see the package docstring.

This is the plain definition of the computation pass the pages describe (SALE,
"What carries the argument": attention is computed only on the selected blocks;
AnchorAttention, "Core claim": only the selected key/value rows are loaded): for a query
row r of head h in query block i, the keys are the tokens named by the kept list of
(batch, KV head of h, i) that satisfy j <= r (causal), and

    z_j = c * q_r . k_j,   O_r = sum_j softmax(z)_j v_j,   LSE_r = log sum_j exp(z_j).

Block lists name key blocks of ``block_k`` tokens; stripe lists name key columns.
"""
from __future__ import annotations

import numpy as np

from .estimate import _f64, softmax_scale, query_block_rows


def _keys_of_list(kept, granularity: str, block_k: int, n: int) -> np.ndarray:
    kept = np.asarray(kept, dtype=np.int64)
    if granularity == "stripe":
        return kept
    if kept.size == 0:
        return kept
    toks = (kept[:, None] * block_k + np.arange(block_k)[None, :]).reshape(-1)
    return toks[toks < n]


def attention_rows(q, k, v, lists, *, block_q: int, block_k: int, granularity: str = "block",
                   rows, scale: float | None = None, kv_of_q=None):
    """Attention for the query blocks ``rows`` = iterable of (b, h, i) (h = query head).

    ``lists``: mapping (b, g, i) -> ascending kept indices (block ids or column ids).
    Returns {(b, h, i): (O [rows, d] float64, LSE [rows] float64)}.
    """
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    c = float(softmax_scale(D, scale))
    if kv_of_q is None:
        kv_of_q = np.arange(Hq) // (Hq // Hkv)
    out = {}
    kcache = {}
    for (b, h, i) in rows:
        g = int(kv_of_q[h])
        if (b, g) not in kcache:
            kcache.clear()
            kcache[(b, g)] = (_f64(k[b, :, g, :]), _f64(v[b, :, g, :]))
        kf, vf = kcache[(b, g)]
        r0, r1 = query_block_rows(i, N, block_q)
        toks = _keys_of_list(lists[(b, g, i)], granularity, block_k, N)
        qb = _f64(q[b, r0:r1, h, :])
        z = c * (qb @ kf[toks].T)                                   # [rows, keys]
        z = np.where(toks[None, :] <= np.arange(r0, r1)[:, None], z, -np.inf)
        m = z.max(axis=1, keepdims=True)
        p = np.exp(z - m)
        s = p.sum(axis=1, keepdims=True)
        o = (p / s) @ vf[toks]
        lse = (m + np.log(s))[:, 0]
        out[(b, h, i)] = (o, lse)
    return out


def attention_all(q, k, v, lists, *, block_q, block_k, granularity="block", scale=None,
                  kv_of_q=None):
    """Full output: O [B, N, Hq, d] float64 and LSE [B, Hq, N] float64."""
    B, N, Hq, D = q.shape
    nqb = -(-N // block_q)
    rows = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(nqb)]
    res = attention_rows(q, k, v, lists, block_q=block_q, block_k=block_k,
                         granularity=granularity, rows=rows, scale=scale, kv_of_q=kv_of_q)
    O = np.empty((B, N, Hq, D))
    LSE = np.empty((B, Hq, N))
    for (b, h, i), (o, lse) in res.items():
        r0, r1 = query_block_rows(i, N, block_q)
        O[b, r0:r1, h, :] = o
        LSE[b, h, r0:r1] = lse
    return O, LSE


def dense_causal_reference_mask(n: int) -> np.ndarray:
    """Boolean [n, n] causal mask (True = attend), for the theta = +inf equivalence."""
    return np.tril(np.ones((n, n), dtype=bool))
