"""GPU parity of anchor-state reuse with column (stripe) lists: the estimate with the state
gives the plain stripe estimate's lists bit for bit and a state within the output bars of the
oracle's attention over each row's anchor region; the prefill resumed from the state over the
oracle's column lists matches the oracle's attention over those lists; over caller-built
column lists (random columns, entries past the block's last row, lists without the anchor
region) it matches the oracle's resume (state merged with the listed columns outside A(r))."""
import numpy as np
import pytest

import oracle
import synth
from helpers import MAX_ABS, MEAN_ABS, compare_lists, compare_outputs, lists_from_ref, log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    import block_sparse_attention_estimate_amd as sa
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sa.load_library()
    return torch.device("cuda:0")


def _upload(lists_np, shape, dev, stride):
    import torch
    import block_sparse_attention_estimate_amd as sa
    B, Hkv, nqb = shape
    counts = np.zeros((B, Hkv, nqb), np.int32)
    idx = np.zeros((B, Hkv, nqb, stride), np.int32)
    for (b, g, i), kept in lists_np.items():
        counts[b, g, i] = kept.size
        idx[b, g, i, :kept.size] = kept
    return sa.Lists(torch.from_numpy(counts).to(dev), torch.from_numpy(idx).to(dev), stride,
                    "stripe")


def _state_errors(st, sref, N, bq):
    so, sl = st.o.float().cpu().numpy(), st.lse.cpu().numpy()
    errs, lerrs = [], []
    for (b, h, i), (oa, la) in sref.items():
        r0, r1 = i * bq, min(N, (i + 1) * bq)
        errs.append(np.abs(so[b, r0:r1, h, :] - oa).ravel())
        lerrs.append(np.abs(sl[b, h, r0:r1] - la))
    return np.concatenate(errs), np.concatenate(lerrs)


@pytest.mark.parametrize("seq,hq,hkv,d,bq,sink,local", [
    (3000, 8, 2, 128, 128, 32, 256),     # the stripe workload's sink and window, ragged tail
    (1500, 4, 1, 64, 64, 32, 256),
    (1300, 8, 2, 128, 128, 0, 100),      # no sink, a short window
    (900, 2, 2, 128, 128, 70, 40),       # sink past one tile, window under one
    (2100, 16, 2, 128, 128, 32, 256),    # 8 heads per KV head
])
def test_stripe_resume_reduced(dev, seq, hq, hkv, d, bq, sink, local):
    import torch
    import block_sparse_attention_estimate_amd as sa
    x = synth.make_prefill("stripe_64k", seq=seq, hq=hq, hkv=hkv, head_dim=d)
    B, N, Hq, D = x.q.shape
    grp = hq // hkv
    theta = np.repeat(np.array([2.0, 3.0, 4.0, 3.5] * 8, np.float32)[:hkv], grp)
    log(f"stripe resume N={N} Hq={Hq} Hkv={hkv} d={D} bq={bq} sink={sink} local={local}")
    q, k, v = to_dev(x.q, dev), to_dev(x.k, dev), to_dev(x.v, dev)
    kw = dict(block_q=bq, block_k=64, sink=sink, local=local)
    plain = sa.estimate_mask(q, k, theta, granularity="stripe", **kw)
    lists, st = sa.estimate_mask_anchor_state(q, k, v, theta, granularity="stripe", **kw)
    torch.cuda.synchronize()
    assert torch.equal(plain.counts, lists.counts)
    c = plain.counts.cpu().numpy().reshape(-1)
    i0 = plain.idx.cpu().numpy().reshape(c.size, -1)
    i1 = lists.idx.cpu().numpy().reshape(c.size, -1)
    for r in range(c.size):
        assert np.array_equal(i0[r, :c[r]], i1[r, :c[r]])
    ref = oracle.estimate_all(x.q, x.k, theta, granularity="stripe", **kw)
    rows_l, entries, flips = compare_lists(lists, ref)
    nqb = -(-N // bq)
    rows = [(0, h, i) for h in range(Hq) for i in range(nqb)]
    sref = oracle.anchor_state_rows(x.q, x.k, x.v, block_q=bq, sink=sink, local=local, rows=rows)
    err, lerr = _state_errors(st, sref, N, bq)
    assert err.max() < MAX_ABS and err.mean() < MEAN_ABS and lerr.max() < 1e-2
    # the resumed prefill under the oracle's lists = attention over those lists
    ol = {key: r["kept"] for key, r in ref.items()}
    dl = _upload(ol, (B, hkv, nqb), dev, N)
    o, lse = sa.sparse_prefill_resume(q, k, v, dl, st, **kw)
    torch.cuda.synchronize()
    O, LSE = oracle.attention_all(x.q, x.k, x.v, lists_from_ref(ref), block_q=bq, block_k=64,
                                  granularity="stripe")
    mx, mean, lmax = compare_outputs(o, lse, O, LSE)
    # and it equals the plain stripe prefill over the same lists within the output bars
    o2, lse2 = sa.sparse_prefill(q, k, v, dl, **kw)
    torch.cuda.synchronize()
    d2 = (o.float() - o2.float()).abs()
    assert d2.max().item() < MAX_ABS and d2.mean().item() < MEAN_ABS
    log(f"  lists equal ({rows_l} rows, {entries} entries, {flips} flips); state "
        f"max|dO|={err.max():.2e}; resumed max|dO|={mx:.2e} mean={mean:.2e} max|dLSE|={lmax:.2e}")


@pytest.mark.parametrize("sink,local", [(32, 256), (0, 64)])
def test_stripe_resume_caller_lists(dev, sink, local):
    """Caller-built column lists (not from the estimate): random columns anywhere (future ones
    too), empty lists, lists of only anchor-region columns and lists without the anchor region;
    the result is the oracle's resume: the state merged with the listed causal columns outside
    each row's anchor region."""
    import torch
    import block_sparse_attention_estimate_amd as sa
    x = synth.make_prefill("stripe_64k", seq=1700, hq=8, hkv=2, head_dim=128)
    B, N, Hq, D = x.q.shape
    bq, Hkv = 128, 2
    nqb = -(-N // bq)
    q, k, v = to_dev(x.q, dev), to_dev(x.k, dev), to_dev(x.v, dev)
    kw = dict(block_q=bq, block_k=64, sink=sink, local=local)
    _, st = sa.estimate_mask_anchor_state(q, k, v, np.full(Hq, 3.0, np.float32),
                                          granularity="stripe", **kw)
    rng = np.random.default_rng(31)
    cl = {}
    for g in range(Hkv):
        for i in range(nqb):
            kind = int(rng.integers(0, 4))
            r0, r1 = i * bq, min(N, (i + 1) * bq)
            if kind == 0:
                kept = np.zeros(0, np.int64)
            elif kind == 1:                          # only the anchor region's columns
                kept = oracle.forced_columns(i, N, bq, sink, local)
            else:                                    # random, incl. future and anchor columns
                kept = np.nonzero(rng.random(N) < rng.uniform(0.02, 0.5))[0]
            cl[(0, g, i)] = np.asarray(kept, np.int64)
    dl = _upload(cl, (B, Hkv, nqb), dev, N)
    o, lse = sa.sparse_prefill_resume(q, k, v, dl, st, **kw)
    torch.cuda.synchronize()
    rows = [(0, h, i) for h in range(Hq) for i in range(nqb)]
    sref = oracle.anchor_state_rows(x.q, x.k, x.v, block_q=bq, sink=sink, local=local, rows=rows)
    res = oracle.resume_rows(x.q, x.k, x.v, cl, sref, block_q=bq, block_k=64, sink=sink,
                             local=local, rows=rows, granularity="stripe")
    og, lg = o.float().cpu().numpy(), lse.cpu().numpy()
    errs, lerrs = [], []
    for (b, h, i), (O, L) in res.items():
        r0, r1 = i * bq, min(N, (i + 1) * bq)
        errs.append(np.abs(og[b, r0:r1, h, :] - O).ravel())
        lerrs.append(np.abs(lg[b, h, r0:r1] - L))
    err, lerr = np.concatenate(errs), np.concatenate(lerrs)
    log(f"  caller column lists resumed: max|dO|={err.max():.2e} mean={err.mean():.2e} "
        f"max|dLSE|={lerr.max():.2e}")
    assert err.max() < MAX_ABS and err.mean() < MEAN_ABS and lerr.max() < 1e-2
