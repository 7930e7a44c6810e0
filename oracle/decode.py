"""Sparse decode: block summaries, forced + top-K block selection, attention over the
selected blocks (oracle, CPU, fp64).

TEST INFRASTRUCTURE -- see the package docstring.

Sources (review pages, cited by title and section):
* SpotAttention: Plug-In Block-Sparse Routing for Pretrained Long-Context Transformers
  (arXiv 2606.22874) -- Figure 2 caption: every past block is scored, the index set I is a
  sink prefix, a recency window and the top-scoring content blocks, and attention runs over
  the gathered K_I, V_I only.  Its learned scorer is replaced here by a training-free one.
* SALE (arXiv 2505.24179) -- "The reading": coarse block-representative schemes score
  one summary per key block; the summary used here is the block's mean key.
* KVpop (arXiv 2607.05061) -- referee minor comment 4: grouped query heads are
  aggregated with max.

Quantised summaries (SpotAttention "Key findings": an INT4 / FP4 selector key cache is 3.5x
smaller at no accuracy cost): each summary row is cut into groups of 32 dims; a group with
a = max |x| gets the scale fp32(a / 7) rounded to bf16 and codes clamp(rint_even(fp32(x *
fp32(7 / a))), -7, 7) (all zero for a = 0); the score then uses scale * code.  Storage
(``pack_q4``) is a layout choice of this library, not the pages'.  4 code bits
per dim plus one 16-bit scale per 32 dims is 4.5 bits per dim instead of 16 (3.56x).  The
FP4 form (``quantize_summary_fp4``) is OCP MXFP4: E2M1 values with one power-of-two scale per
32 dims, 4.25 bits per dim (3.76x).

Readings: the summary is the mean of the block's cached keys (fp64 sum, fp64 division,
rounded to fp32 and then to bf16, round to nearest even); the block score is the max over
the group's query heads of c * q_h . kbar_J; the forced set is every block overlapping the
sink tokens [0, sink) or the recency window [L - local, L - 1]; the remaining K - |F|
blocks are the highest scores, ties to the lower block index; the query sits at position
L - 1 and sees every cached token.

Per-query budget (SpotAttention abstract and Figure 2 caption: a dual top-p rule reads the
budget from the selector's own distribution over blocks, and I holds the sink prefix, the
recency window and the top-p content blocks; Figure 7 plots the cumulative mass of the blocks
kept in descending score order).  The rule is named but not spelled out; the reading here:
the distribution is pi_J = exp(score_J) / sum_J' exp(score_J') over the blocks of the cache,
the forced blocks count first, and then content blocks are added in (score desc, block asc)
order until the cumulative share reaches top_p; the selection never exceeds K blocks in all
(the second bound of the rule).  top_p = 0 keeps the fixed K.
"""
from __future__ import annotations

import numpy as np

from .estimate import _f64, softmax_scale
from .estimate_sale import E2M1_GRID, dequantize_mxfp4, quantize_mxfp4

AMBIGUITY_BAND = 1e-3
# a budget is ambiguous when a cumulative share next to the decision lies this close to top_p
TOP_P_BAND = 1e-4


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def block_summary(k_cache, cache_len, block_k: int) -> np.ndarray:
    """kbar[b, J, g, :] as bf16 bit patterns; blocks past the cache length are zero."""
    B, L, Hkv, D = k_cache.shape
    nkb = -(-L // block_k)
    out = np.zeros((B, nkb, Hkv, D), dtype=np.uint16)
    for b in range(B):
        lb = int(cache_len[b])
        kf = _f64(k_cache[b, :lb])                                 # [lb, Hkv, D]
        for J in range(-(-lb // block_k)):
            a, e = J * block_k, min(lb, (J + 1) * block_k)
            mean = kf[a:e].sum(axis=0) / float(e - a)              # fp64
            out[b, J] = _f32_to_bf16_bits(mean.astype(np.float32))
    return out


Q4_GROUP = 32


def quantize_summary_q4(kbar: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """kbar bf16 bits [..., D] -> (codes int8 [..., D] in [-7, 7], scales bf16 bits
    [..., D / 32])."""
    x = _f64(kbar).astype(np.float32)
    shp = x.shape[:-1] + (x.shape[-1] // Q4_GROUP, Q4_GROUP)
    xg = x.reshape(shp)
    a = np.abs(xg).max(axis=-1)                                     # fp32 [..., D/32]
    nz = a > 0
    inv = np.where(nz, np.float32(7.0) / np.where(nz, a, np.float32(1.0)), np.float32(0.0))
    inv = inv.astype(np.float32)
    y = (xg * inv[..., None]).astype(np.float32)                  # one fp32 rounding
    codes = np.clip(np.rint(y), -7, 7).astype(np.int8)
    scale = np.where(nz, (a / np.float32(7.0)).astype(np.float32), np.float32(0.0))
    return codes.reshape(x.shape), _f32_to_bf16_bits(scale.astype(np.float32))


def dequantize_summary_q4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """scale * code as float64 [..., D] (exact: a bf16 scale times a small integer)."""
    c = codes.astype(np.float64)
    shp = c.shape[:-1] + (c.shape[-1] // Q4_GROUP, Q4_GROUP)
    return (c.reshape(shp) * _f64(scales)[..., None]).reshape(c.shape)


def pack_q4(codes: np.ndarray) -> np.ndarray:
    """Storage of the codes: offset-binary nibbles u = code + 8 (1 .. 15); each 32-bit
    little-endian word holds 8 consecutive dims, dim 2j in nibble j and dim 2j + 1 in nibble
    j + 4 (j = 0..3).  Returns uint8 [..., D / 2]."""
    u = (codes.astype(np.int64) + 8).astype(np.uint32)
    shp = u.shape[:-1] + (u.shape[-1] // 8, 8)
    u = u.reshape(shp)
    w = np.zeros(shp[:-1], dtype=np.uint32)
    for j in range(4):
        w |= u[..., 2 * j] << np.uint32(4 * j)
        w |= u[..., 2 * j + 1] << np.uint32(4 * (j + 4))
    return w.view(np.uint8).reshape(codes.shape[:-1] + (codes.shape[-1] // 2,))


def quantize_summary_fp4(kbar: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """FP4 summaries (the page's other 4-bit format: FP4 microscale), read as OCP MXFP4: each
    group of 32 dims shares the exponent e = floor(log2 max|x|) - 2 and each dim is an E2M1
    value (the MXFP4 quantiser of the relative estimator).  kbar bf16 bits [..., D] ->
    (values float64 [..., D] on the signed E2M1 grid, exponents int [..., D / 32]); the
    summary is read as values * 2 ** e."""
    return quantize_mxfp4(_f64(kbar).astype(np.float32))


def dequantize_summary_fp4(vals: np.ndarray, exps: np.ndarray) -> np.ndarray:
    return dequantize_mxfp4(vals, exps)


def pack_fp4(kbar: np.ndarray, vals: np.ndarray, exps: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Storage of FP4 summaries (a layout choice of this library): per dim the E2M1 nibble
    (magnitude index into the grid 0, 0.5, 1, 1.5, 2, 3, 4, 6 in bits 0-2, the sign bit of the
    summary value -- negative zero included -- in bit 3), dim 2k in the low and 2k + 1 in the
    high nibble of byte k; per 32 dims the E8M0 byte e + 127.
    Returns (codes uint8 [..., D / 2], exps uint8 [..., D / 32])."""
    mag = np.searchsorted(E2M1_GRID, np.abs(vals)).astype(np.uint8)   # exact grid values
    sign = np.signbit(_f64(kbar).astype(np.float32)).astype(np.uint8)
    nib = mag | (sign << 3)
    codes = nib[..., 0::2] | (nib[..., 1::2] << 4)
    return codes.astype(np.uint8), (np.asarray(exps) + 127).astype(np.uint8)


def decode_forced(n_blocks: int, length: int, block_k: int, sink: int, local: int) -> np.ndarray:
    J = np.arange(n_blocks)
    sink_hit = J * block_k < sink
    lo = max(0, length - local)
    win_hit = (J + 1) * block_k - 1 >= lo
    return J[sink_hit | win_hit]


def top_p_budget(score: np.ndarray, is_forced: np.ndarray, top_p: float):
    """Number of content blocks the top-p rule adds to the forced set: the fewest, taken in
    (score desc, block asc) order, that bring forced share + their share of
    pi = softmax(score) to at least top_p.  Returns (k, order, ambiguous): order is the
    content blocks in that order; ambiguous is True when the cumulative share after k - 1 or
    after k blocks lies within TOP_P_BAND of top_p."""
    score = np.asarray(score, dtype=np.float64)
    w = np.exp(score - score.max())
    z = w.sum()
    order = sorted(np.nonzero(~is_forced)[0].tolist(), key=lambda J: (-score[J], J))
    cum = [w[is_forced].sum() / z]                  # share after 0, 1, 2, ... content blocks
    for J in order:
        cum.append(cum[-1] + w[J] / z)
    k = 0
    while k < len(order) and cum[k] < top_p:
        k += 1
    near = [cum[k]] + ([cum[k - 1]] if k > 0 else [])
    ambiguous = any(abs(v - top_p) < TOP_P_BAND for v in near)
    return k, np.array(order, dtype=np.int64), ambiguous


def decode_select(q, kbar, cache_len, *, block_k: int, top_k: int, sink: int, local: int,
                  scale: float | None = None, kv_of_q=None, top_p: float = 0.0) -> dict:
    """Per (b, g): ascending selected block ids, the scores and the ambiguous blocks
    (non-forced blocks whose score lies within the band of the selection boundary).  With
    top_p > 0 the number of content blocks is the top-p budget capped at K - |F|; the entry
    also holds the budget ("budget"), whether it is ambiguous ("budget_ambiguous") and the
    content blocks in selection order ("order")."""
    B, Hq, D = q.shape
    Hkv = kbar.shape[2]
    c = float(softmax_scale(D, scale))
    if kv_of_q is None:
        kv_of_q = np.arange(Hq) // (Hq // Hkv)
    kv_of_q = np.asarray(kv_of_q)
    out = {}
    for b in range(B):
        lb = int(cache_len[b])
        nkb = -(-lb // block_k)
        for g in range(Hkv):
            heads = np.nonzero(kv_of_q == g)[0]
            kb = _f64(kbar[b, :nkb, g, :])                          # [nkb, D]
            # (kbar may be bf16 bits or float values, e.g. dequantised q4 summaries)
            qh = _f64(q[b, heads, :])                               # [heads, D]
            score = (c * (qh @ kb.T)).max(axis=0)                   # [nkb]
            forced = decode_forced(nkb, lb, block_k, sink, local)
            if top_p > 0:
                is_f = np.zeros(nkb, dtype=bool)
                is_f[forced] = True
                k, order, bamb = top_p_budget(score, is_f, top_p)
                n_pick = min(k, max(0, top_k - forced.size))
                sel = np.union1d(forced, order[:n_pick])
                rest = order
                if 0 < n_pick < order.size:
                    bound = score[order[n_pick - 1]]
                    amb = rest[np.abs(score[rest] - bound) < AMBIGUITY_BAND]
                else:
                    amb = np.zeros(0, dtype=np.int64)
                out[(b, g)] = dict(selected=sel.astype(np.int32), score=score,
                                   forced=forced.astype(np.int32), ambiguous=amb.astype(np.int32),
                                   budget=n_pick, budget_uncapped=k,
                                   budget_ambiguous=bool(bamb) and n_pick == k, order=order)
                continue
            if nkb <= top_k:
                sel = np.arange(nkb)
                amb = np.zeros(0, dtype=np.int64)
            else:
                is_f = np.zeros(nkb, dtype=bool)
                is_f[forced] = True
                rest = np.nonzero(~is_f)[0]
                n_pick = max(0, top_k - forced.size)
                order = sorted(rest.tolist(), key=lambda J: (-score[J], J))
                pick = np.array(order[:n_pick], dtype=np.int64)
                sel = np.union1d(forced, pick)
                if n_pick > 0:
                    bound = score[order[n_pick - 1]]
                    amb = rest[np.abs(score[rest] - bound) < AMBIGUITY_BAND]
                else:
                    amb = np.zeros(0, dtype=np.int64)
            out[(b, g)] = dict(selected=sel.astype(np.int32), score=score,
                               forced=forced.astype(np.int32), ambiguous=amb.astype(np.int32))
    return out


def decode_attention(q, k_cache, v_cache, cache_len, selected, *, block_k: int,
                     scale: float | None = None, kv_of_q=None):
    """O [B, Hq, D] float64 and LSE [B, Hq] over the tokens of the selected blocks."""
    B, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    c = float(softmax_scale(D, scale))
    if kv_of_q is None:
        kv_of_q = np.arange(Hq) // (Hq // Hkv)
    O = np.empty((B, Hq, D))
    LSE = np.empty((B, Hq))
    for b in range(B):
        lb = int(cache_len[b])
        for h in range(Hq):
            g = int(kv_of_q[h])
            sel = np.asarray(selected[(b, g)], dtype=np.int64)
            toks = (sel[:, None] * block_k + np.arange(block_k)[None, :]).reshape(-1)
            toks = toks[toks < lb]
            kf = _f64(k_cache[b, toks, g, :])
            vf = _f64(v_cache[b, toks, g, :])
            z = c * (kf @ _f64(q[b, h, :]))
            m = z.max()
            p = np.exp(z - m)
            s = p.sum()
            O[b, h] = (p / s) @ vf
            LSE[b, h] = m + np.log(s)
    return O, LSE
