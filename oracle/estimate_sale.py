"""Element-wise low-bit estimation with the relative attention score (oracle, CPU, fp64).

TEST INFRASTRUCTURE -- see the package docstring.

Source: SALE: Low-bit Estimation for Efficient Sparse Attention in Long-context LLM
Prefilling (arXiv 2505.24179).
* "What carries the argument": every query-key pair is estimated from low-bit Q and K
  (S~[i, j]); the relative attention score is P~[i, j] = exp(S~[i, j] - em_i) / el_i with
  em_i and el_i the maximum and the sum of exp(S~ - em_i) over row i's sink-local area (the
  first 32 tokens and the most recent, up to 256, tokens); a block is skipped only when every
  estimate inside it falls below the per-head threshold tau.
* Referee major comment 1: the log form of that test is S~[i, j] >= ln(tau * el_i) + em_i
  (the printed Eq. 4 misplaces em_i).
* "Assumptions & free parameters": tau per head, bq = 64 and bk = 32 on the pages (the
  block sizes here are the caller's).

Readings (the design notes of the repository list them with their reasons):
* theta = -ln tau, so the test is S~[r, j] - LSE_r >= -theta with LSE_r = em_r + ln el_r,
  the log-sum-exp of S~ over row r's area; the margin of a (query block, key block) pair is
  max over its rows r and causal keys j of S~[r, j] - LSE_r, plus theta of the head;
* the sink-local area of row r is the token set {j < sink} U {max(0, r - local + 1) <= j <= r}
  (each key once), the same region as the pooled estimator's anchor;
* low bit is int8 (the Q8 rule of ``quantize_q8``) with one scale per query row and one per
  key tile of ``block_k`` keys; S~ = fp32(D) * fp32(fp32(s_q * s_K) * c) with D the exact
  integer dot product; em, el and LSE are evaluated in fp64 from those fp32 values;
* grouped query heads: the union (max of margins) over the group, as for the pooled form;
  forced blocks, candidates and the ambiguity band are those of ``estimate_rows``.

4-bit variant (``lowbit="mxfp4"``; the pages' estimate is 4-bit): Q rows and K rows are
quantised to MXFP4 as the OCP Microscaling Formats (MX) v1.0 specification defines it -- per
block of 32 consecutive head dims a shared power-of-two scale 2^e with e = floor(log2(max|x|))
- 2 (the largest E2M1 exponent) clamped to [-127, 127], and elements E2M1 = round-to-nearest-
even of x / 2^e onto {0, 0.5, 1, 1.5, 2, 3, 4, 6} with saturation at 6.  The dot product of
the dequantised values is exact in fp64; S~ = fp32(fp32(dot) * c).
"""
from __future__ import annotations

import numpy as np

from .estimate import (AMBIGUITY_BAND, _f64, forced_blocks, quantize_key_tiles, quantize_q8,
                       query_block_rows, softmax_scale)


E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
MX_BLOCK = 32


def quantize_mxfp4(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """MXFP4 per block of 32 along the last axis.  Returns (values, exps): values are the
    signed E2M1 numbers [..., d] (before scaling), exps the shared exponents [..., d / 32]
    (int); the dequantised tensor is values * 2.0 ** exps (repeated over each block)."""
    x = np.asarray(x, dtype=np.float32)
    shp = x.shape
    xb = x.reshape(shp[:-1] + (shp[-1] // MX_BLOCK, MX_BLOCK)).astype(np.float64)
    amax = np.abs(xb).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))).astype(np.int64) - 2
    e = np.where(amax > 0, e, -127)
    e = np.clip(e, -127, 127)
    y = np.abs(xb) / np.ldexp(1.0, e)[..., None]           # exact: a power-of-two scale
    # round to nearest on the E2M1 grid, ties to the even code (mantissa bit 0)
    idx = np.searchsorted(E2M1_GRID, y, side="left")
    idx = np.clip(idx, 1, len(E2M1_GRID) - 1)
    lo, hi = E2M1_GRID[idx - 1], E2M1_GRID[idx]
    d_lo, d_hi = y - lo, hi - y
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((idx % 2) == 0))
    code = np.where(pick_hi, idx, idx - 1)
    code = np.where(y >= E2M1_GRID[-1], len(E2M1_GRID) - 1, code)       # saturate at 6
    vals = np.sign(xb) * E2M1_GRID[code]
    return vals.reshape(shp), e


def dequantize_mxfp4(vals: np.ndarray, exps: np.ndarray) -> np.ndarray:
    return vals * np.repeat(np.ldexp(1.0, exps), MX_BLOCK, axis=-1)


def area_mask(r0: int, r1: int, n_keys: int, sink: int, local: int) -> np.ndarray:
    """[n_keys, r1 - r0] bool: key j lies in row r's sink-local area."""
    j = np.arange(n_keys)[:, None]
    r = np.arange(r0, r1)[None, :]
    return ((j < sink) | ((j >= r - local + 1) & (j <= r))) & (j <= r)


def relative_scores(s_hat: np.ndarray, r0: int, sink: int, local: int) -> np.ndarray:
    """s_hat [n_keys, rows] (keys 0 .. n_keys-1, rows r0 ..) -> S~ - LSE_r over causal keys
    (-inf elsewhere), LSE_r the log-sum-exp over the row's sink-local area."""
    n_keys, rows = s_hat.shape
    area = area_mask(r0, r0 + rows, n_keys, sink, local)
    em = np.where(area, s_hat, -np.inf).max(axis=0)                  # [rows]
    el = np.where(area, np.exp(s_hat - em[None, :]), 0.0).sum(axis=0)
    lse = em + np.log(el)
    causal = np.arange(n_keys)[:, None] <= np.arange(r0, r0 + rows)[None, :]
    return np.where(causal, s_hat - lse[None, :], -np.inf)


def estimate_rows_sale(q, k, theta, *, block_q: int, block_k: int, sink: int, local: int,
                       rows, scale: float | None = None, kv_of_q=None, quantized: bool = True,
                       keep_margins: bool = True, per_head: bool = False,
                       lowbit: str = "int8") -> dict:
    """Kept block lists of the rows ``rows`` = iterable of (b, g, i) under the element-wise
    estimate; the result has the layout of ``estimate_rows`` (block granularity).  lowbit:
    "int8" (rows of Q and tiles of K) or "mxfp4" (32-dim blocks of Q and K rows)."""
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    c = softmax_scale(D, scale)
    theta = np.asarray(theta, dtype=np.float64).reshape(Hq)
    if kv_of_q is None:
        kv_of_q = np.arange(Hq) // (Hq // Hkv)
    kv_of_q = np.asarray(kv_of_q)
    out = {}
    cache_key, kf, kq64, sk = None, None, None, None
    for (b, g, i) in rows:
        if cache_key != (b, g):
            kf = _f64(k[b, :, g, :])
            if lowbit == "mxfp4":
                kq64 = dequantize_mxfp4(*quantize_mxfp4(kf.astype(np.float32)))
            else:
                kq, sk = quantize_key_tiles(kf, block_k)
                kq64 = kq.astype(np.float64)
            cache_key = (b, g)
        r0, r1 = query_block_rows(i, N, block_q)
        e = r1 - 1
        ncand = e // block_k + 1
        tile = np.arange(e + 1) // block_k
        heads = np.nonzero(kv_of_q == g)[0]
        margins = []
        for h in heads:
            qb = _f64(q[b, r0:r1, h, :])
            if quantized and lowbit == "mxfp4":
                qd = dequantize_mxfp4(*quantize_mxfp4(qb.astype(np.float32)))
                dots = kq64[: e + 1] @ qd.T                              # exact in fp64
                s_hat = (dots.astype(np.float32) * c).astype(np.float32).astype(np.float64)
            elif quantized:
                qq, sq = quantize_q8(qb.astype(np.float32), axis=1)      # per query row
                dots = kq64[: e + 1] @ qq.astype(np.float64).T           # exact integers
                mult = ((sq[None, :] * sk[tile][:, None]).astype(np.float32) * c).astype(np.float32)
                s_hat = (dots.astype(np.float32) * mult).astype(np.float32).astype(np.float64)
            else:
                s_hat = float(c) * (kf[: e + 1] @ qb.T)
            rel = relative_scores(s_hat, r0, sink, local)                # [keys, rows]
            pad = np.full((ncand * block_k, r1 - r0), -np.inf)
            pad[: e + 1] = rel
            E = pad.reshape(ncand, block_k * (r1 - r0)).max(axis=1)
            margins.append(E + theta[h])
        mh = np.stack(margins)
        mg = mh.max(axis=0)
        forced = forced_blocks(i, N, block_q, block_k, sink, local)
        cand = np.arange(ncand)
        is_forced = np.zeros(ncand, dtype=bool)
        is_forced[forced] = True
        keep = is_forced | (mg >= 0)
        amb = (~is_forced) & (np.abs(mg) < AMBIGUITY_BAND)
        rec = dict(kept=cand[keep].astype(np.int32), forced=forced.astype(np.int32),
                   ambiguous=cand[amb].astype(np.int32), n_candidates=int(ncand))
        if keep_margins:
            rec["margin"] = mg
        if per_head:
            rec["kept_per_head"] = [cand[is_forced | (m >= 0)].astype(np.int32) for m in mh]
        out[(b, g, i)] = rec
    return out


def estimate_all_sale(q, k, theta, *, block_q, block_k, sink, local, scale=None, kv_of_q=None,
                      quantized=True, keep_margins=True, per_head=False, lowbit="int8") -> dict:
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    nqb = -(-N // block_q)
    rows = [(b, g, i) for b in range(B) for g in range(Hkv) for i in range(nqb)]
    return estimate_rows_sale(q, k, theta, block_q=block_q, block_k=block_k, sink=sink,
                              local=local, rows=rows, scale=scale, kv_of_q=kv_of_q,
                              quantized=quantized, keep_margins=keep_margins, per_head=per_head,
                              lowbit=lowbit)
