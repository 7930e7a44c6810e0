"""Shared helpers for the GPU parity tests: host<->device marshalling and comparisons."""
import sys
import time

import numpy as np

import oracle

MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def bf16_to_np(t):
    import torch
    return t.float().cpu().numpy().astype(np.float64)


def compare_lists(gpu_lists, ref: dict):
    """Kept lists must agree exactly except entries the oracle marks ambiguous (|margin| within
    the band of the threshold).  Returns (rows checked, entries compared, ambiguous flips)."""
    counts = gpu_lists.counts.cpu().numpy()
    idx = gpu_lists.idx.cpu().numpy()
    n_entries = 0
    flips = 0
    for (b, g, i), r in ref.items():
        c = int(counts[b, g, i])
        assert c <= gpu_lists.stride, ("overflow", (b, g, i), c)
        got = idx[b, g, i, :c]
        assert np.all(np.diff(got) > 0), ("not ascending", (b, g, i))
        diff = set(got.tolist()) ^ set(r["kept"].tolist())
        amb = set(r["ambiguous"].tolist())
        bad = diff - amb
        assert not bad, ("list mismatch", (b, g, i), sorted(bad)[:10])
        flips += len(diff)
        n_entries += len(r["kept"])
    return len(ref), n_entries, flips


def lists_from_ref(ref: dict):
    return {key: r["kept"] for key, r in ref.items()}


def upload_lists(ref: dict, shape, dev, granularity, stride):
    """Oracle lists -> device Lists (the attention parity runs under the oracle's mask)."""
    import torch
    import block_sparse_attention_estimate_amd as sa
    B, Hkv, nqb = shape
    counts = np.zeros((B, Hkv, nqb), dtype=np.int32)
    idx = np.zeros((B, Hkv, nqb, stride), dtype=np.int32)
    for (b, g, i), r in ref.items():
        k = r["kept"]
        counts[b, g, i] = len(k)
        idx[b, g, i, :len(k)] = k
    return sa.Lists(torch.from_numpy(counts).to(dev), torch.from_numpy(idx).to(dev), stride,
                    granularity)


def compare_outputs(o_gpu, lse_gpu, O_ref, LSE_ref, rows=None):
    """rows: optional list of (b, h, r0, r1) slices; default all."""
    o = bf16_to_np(o_gpu)
    lse = lse_gpu.cpu().numpy().astype(np.float64) if lse_gpu is not None else None
    if rows is None:
        err = np.abs(o - O_ref)
        lerr = np.abs(lse - LSE_ref) if lse is not None else np.zeros(1)
    else:
        errs, lerrs = [], []
        for (b, h, r0, r1, oref, lref) in rows:
            errs.append(np.abs(o[b, r0:r1, h, :] - oref).ravel())
            if lse is not None:
                lerrs.append(np.abs(lse[b, h, r0:r1] - lref))
        err = np.concatenate(errs)
        lerr = np.concatenate(lerrs) if lerrs else np.zeros(1)
    assert np.isfinite(err).all()
    assert err.max() < MAX_ABS, ("max abs", err.max())
    assert err.mean() < MEAN_ABS, ("mean abs", err.mean())
    assert lerr.max() < 1e-2, ("lse", lerr.max())
    return float(err.max()), float(err.mean()), float(lerr.max())


def oracle_estimate_for(x, theta, rows=None, **over):
    kw = dict(block_q=x.block_q, block_k=x.block_k, sink=x.sink, local=x.local,
              granularity=x.granularity)
    kw.update(over)
    if rows is None:
        return oracle.estimate_all(x.q, x.k, theta, **kw)
    return oracle.estimate_rows(x.q, x.k, theta, rows=rows, **kw)


def check_topp_selection(sel_np, ref, band=1e-3):
    """GPU selection under a top-p budget against the oracle's: each (b, g) selects its forced
    blocks plus k content blocks, k equal to the oracle's budget (or one off where the oracle
    flags that budget ambiguous), and those are the first k of the oracle's (score desc, block
    asc) order except blocks whose score lies within `band` of the k-th.  Returns
    ({(b, g): selected}, number of budgets one off, number of exchanged blocks)."""
    used, off, flips = {}, 0, 0
    for (b, g), r in ref.items():
        row = sel_np[b, g]
        n = int((row >= 0).sum())
        got = row[:n]
        assert (row[n:] == -1).all() and np.all(np.diff(got) > 0), (b, g)
        k_gpu = n - r["forced"].size
        if k_gpu != r["budget"]:
            assert r["budget_ambiguous"] and abs(k_gpu - r["budget"]) <= 1, \
                ((b, g), k_gpu, r["budget"])
            off += 1
        order, score = r["order"], r["score"]
        expect = set(r["forced"].tolist()) | set(order[:k_gpu].tolist())
        diff = set(got.tolist()) ^ expect
        if diff:
            assert k_gpu > 0, ((b, g), sorted(diff))
            bound = score[order[k_gpu - 1]]
            amb = {int(J) for J in order if abs(score[J] - bound) < band}
            assert diff <= amb, ((b, g), sorted(diff))
            flips += len(diff)
        used[(b, g)] = got
    return used, off, flips
