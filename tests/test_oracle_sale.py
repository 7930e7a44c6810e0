"""Pins of the oracle's element-wise estimator with the relative attention score (CPU).

* brute force: the literal relative score P~ = exp(S~ - em) / el (exponentials and a
  division, not the log form), a block kept when any causal P~ in it reaches tau =
  exp(-theta) -- pure Python loops on tiny inputs, quantised and unquantised;
* closed form: with every key equal, S~ is constant along a row, so P~ = 1/|area| and a
  block of rows whose areas all hold sink + local keys is kept exactly when
  theta >= ln(sink + local);
* invariants: adding one vector to every key shifts a row's scores by a constant, which the
  relative score cancels (unquantised); theta-nesting; theta = +inf keeps every causal
  block, -inf only the forced ones.
"""
import math

import numpy as np
import pytest

import oracle
from oracle.estimate import quantize_key_tiles, quantize_q8
from oracle.estimate_sale import dequantize_mxfp4, quantize_mxfp4


def _brute(q, k, theta, *, block_q, block_k, sink, local, quantized, lowbit="int8"):
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    c = float(np.float32(1.0 / math.sqrt(D)))
    nqb = -(-N // block_q)
    out = {}
    for b in range(B):
        for g in range(Hkv):
            kf = k[b, :, g, :].astype(np.float64)
            if quantized and lowbit == "mxfp4":
                kd = dequantize_mxfp4(*quantize_mxfp4(kf.astype(np.float32)))
            elif quantized:
                kq, sk = quantize_key_tiles(kf, block_k)
            for i in range(nqb):
                r0, r1 = i * block_q, min(N, (i + 1) * block_q)
                keep = set()
                for h in range(g * G, (g + 1) * G):
                    tau = math.exp(-theta[h])
                    for r in range(r0, r1):
                        qr = q[b, r, h, :].astype(np.float64)
                        if quantized and lowbit == "mxfp4":
                            qd = dequantize_mxfp4(*quantize_mxfp4(qr.astype(np.float32)[None, :]))[0]
                        elif quantized:
                            qq, sq = quantize_q8(qr.astype(np.float32)[None, :], axis=1)
                            qi = [int(v) for v in qq[0]]
                        s = []
                        for j in range(r + 1):
                            if quantized and lowbit == "mxfp4":
                                dot = sum(qd[t] * kd[j, t] for t in range(D))   # exact
                                s.append(float(np.float32(np.float32(dot) * np.float32(c))))
                            elif quantized:
                                dot = sum(qi[t] * int(kq[j, t]) for t in range(D))
                                mult = np.float32(np.float32(sq[0] * sk[j // block_k]) * np.float32(c))
                                s.append(float(np.float32(np.float32(dot) * mult)))
                            else:
                                s.append(c * sum(qr[t] * kf[j, t] for t in range(D)))
                        area = [j for j in range(r + 1) if j < sink or j >= r - local + 1]
                        em = max(s[j] for j in area)
                        el = sum(math.exp(s[j] - em) for j in area)
                        for j in range(r + 1):
                            if math.exp(s[j] - em) / el >= tau:
                                keep.add(j // block_k)
                forced = set(oracle.forced_blocks(i, N, block_q, block_k, sink, local).tolist())
                out[(b, g, i)] = sorted(keep | forced)
    return out


@pytest.mark.parametrize("quantized,lowbit", [(False, "int8"), (True, "int8"), (True, "mxfp4")])
@pytest.mark.parametrize("seed", [0, 1])
def test_brute_force_literal_relative_score(quantized, lowbit, seed):
    rng = np.random.default_rng(seed)
    B, N, Hq, Hkv, D = 1, 150, 4, 2, 32
    q = rng.normal(size=(B, N, Hq, D)).astype(np.float32)
    k = rng.normal(size=(B, N, Hkv, D)).astype(np.float32)
    k[:, 100:103] += 2.5 * q[:, 140:143, ::2]            # a few strong keys
    kw = dict(block_q=32, block_k=16, sink=8, local=40)
    for th in [1.5, 3.0, 4.5]:
        theta = np.array([th, th + 0.7, th - 0.4, th + 0.2])
        ref = oracle.estimate_all_sale(q, k, theta, quantized=quantized, lowbit=lowbit, **kw)
        bf = _brute(q, k, theta, quantized=quantized, lowbit=lowbit, **kw)
        for key, r in ref.items():
            diff = set(r["kept"].tolist()) ^ set(bf[key])
            assert diff <= set(r["ambiguous"].tolist()), (key, th, sorted(diff))


@pytest.mark.parametrize("quantized", [False, True])
def test_equal_keys_closed_form(quantized):
    rng = np.random.default_rng(3)
    B, N, Hq, Hkv, D = 1, 1024, 2, 1, 32
    sink, local, bq, bk = 32, 256, 64, 64
    q = rng.normal(size=(B, N, Hq, D)).astype(np.float32)
    k = np.broadcast_to(rng.normal(size=(1, 1, 1, D)), (B, N, Hkv, D)).astype(np.float32).copy()
    # query blocks from 384 on: every row's area is the 32 sink + 256 local keys
    crit = math.log(sink + local)
    for dth, want_all in [(-0.01, False), (0.01, True)]:
        ref = oracle.estimate_all_sale(q, k, np.full(Hq, crit + dth), block_q=bq, block_k=bk,
                                       sink=sink, local=local, quantized=quantized)
        for (b, g, i), r in ref.items():
            if i * bq < 384:
                continue
            if want_all:
                assert r["kept"].size == r["n_candidates"]
            else:
                assert np.array_equal(r["kept"], r["forced"])


def test_key_shift_invariance_unquantized():
    rng = np.random.default_rng(4)
    B, N, Hq, Hkv, D = 1, 600, 4, 1, 32
    q = rng.normal(size=(B, N, Hq, D))
    k = rng.normal(size=(B, N, Hkv, D))
    u = 3.0 * rng.normal(size=(D,))
    kw = dict(block_q=64, block_k=64, sink=32, local=128, quantized=False)
    a = oracle.estimate_all_sale(q, k, np.full(Hq, 3.0), **kw)
    s = oracle.estimate_all_sale(q, k + u, np.full(Hq, 3.0), **kw)
    for key in a:
        fin = np.isfinite(a[key]["margin"])
        assert np.array_equal(fin, np.isfinite(s[key]["margin"]))
        assert np.allclose(a[key]["margin"][fin], s[key]["margin"][fin], atol=1e-9)


def test_theta_nesting_and_extremes():
    rng = np.random.default_rng(6)
    B, N, Hq, Hkv, D = 1, 900, 4, 2, 32
    q = rng.normal(size=(B, N, Hq, D)).astype(np.float32)
    k = rng.normal(size=(B, N, Hkv, D)).astype(np.float32)
    kw = dict(block_q=64, block_k=64, sink=32, local=128)
    prev = None
    for th in [-np.inf, 1.0, 3.0, 5.0, 7.0, np.inf]:
        ref = oracle.estimate_all_sale(q, k, np.full(Hq, th), **kw)
        for key, r in ref.items():
            kept = set(r["kept"].tolist())
            assert set(r["forced"].tolist()) <= kept
            if th == np.inf:
                assert len(kept) == r["n_candidates"]
            if th == -np.inf:
                assert kept == set(r["forced"].tolist())
            if prev is not None:
                assert prev[key] <= kept
        prev = {key: set(r["kept"].tolist()) for key, r in ref.items()}


def test_relative_scores_row_normalisation():
    # over each row's area the relative scores exp(S~ - LSE) sum to one
    rng = np.random.default_rng(8)
    s = rng.normal(0, 3, size=(300, 40))
    r0 = 260
    rel = oracle.relative_scores(s, r0, sink=32, local=100)
    from oracle.estimate_sale import area_mask
    area = area_mask(r0, r0 + 40, 300, 32, 100)
    tot = np.where(area, np.exp(rel), 0.0).sum(axis=0)
    assert np.allclose(tot, 1.0, atol=1e-12)
