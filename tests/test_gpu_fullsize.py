"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

The oracle recomputes the lists row by row: every row at 32K, 128K and the 64K stripe
workload, sampled rows for the element-wise estimators; attention parity is checked on
sampled query blocks whose GPU list equals the oracle's list (the oracle's list is the
attention input; rows whose lists differ only by ambiguous entries are counted)."""
import numpy as np
import pytest

import oracle
import synth
from helpers import MAX_ABS, MEAN_ABS, check_topp_selection, compare_lists, log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    import block_sparse_attention_estimate_amd as sa
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sa.load_library()
    return torch.device("cuda:0")


_RUN = {}


def _gpu_run(dev, name, estimator, reuse, theta, seed):
    """The GPU estimate + attention of one workload, kept for the tests that follow (the
    every-row tests check one KV head each against the same run)."""
    import torch
    import block_sparse_attention_estimate_amd as sa
    key = (name, estimator, reuse, theta, seed)
    if key in _RUN:
        return _RUN[key]
    _RUN.clear()
    log(f"generating {name}")
    x = synth.make_prefill(name, seed=seed)
    if theta is not None:
        x.theta = np.full(x.q.shape[2], theta, np.float32)
    q, k, v = to_dev(x.q, dev), to_dev(x.k, dev), to_dev(x.v, dev)
    kw = dict(block_q=x.block_q, block_k=x.block_k, sink=x.sink, local=x.local)
    stride = 8192 if x.granularity == "stripe" else None
    st = None
    if reuse:
        lists, st = sa.estimate_mask_anchor_state(q, k, v, x.theta, granularity=x.granularity,
                                                  stride=stride, **kw)
        o, lse = sa.sparse_prefill_resume(q, k, v, lists, st, **kw)
    else:
        lists = sa.estimate_mask(q, k, x.theta, granularity=x.granularity, stride=stride,
                                 estimator=estimator, **kw)
        o, lse = sa.sparse_prefill(q, k, v, lists, **kw)
    torch.cuda.synchronize()
    assert not lists.overflowed()
    run = dict(x=x, lists=lists, o=o.float().cpu(), lse=lse.cpu().numpy(),
               st=None if st is None else (st.o.float().cpu().numpy(), st.lse.cpu().numpy()))
    del q, k, v, o, lse, st
    _RUN[key] = run
    return run


def _prefill_parity(dev, name, n_rows=None, n_attn=12, seed=0, estimator="pooled", reuse=False,
                    theta=None, groups=None):
    """Lists of `n_rows` sampled rows (None: every row of the KV heads in `groups`, default
    all) against the oracle, and the attention of `n_attn` query blocks among them."""
    run = _gpu_run(dev, name, estimator, reuse, theta, seed)
    x, lists = run["x"], run["lists"]
    B, N, Hq, D = x.q.shape
    Hkv = x.k.shape[2]
    G = Hq // Hkv
    nqb = -(-N // x.block_q)
    groups = list(range(Hkv)) if groups is None else list(groups)
    rng = np.random.default_rng(seed + 7 + 101 * groups[0])
    if n_rows is None:
        rows = [(0, g, i) for g in groups for i in range(nqb)]
    else:
        gi = set()
        for g in groups:                         # first, last and random query blocks
            gi.add((g, 0))
            gi.add((g, nqb - 1))
        while len(gi) < n_rows:
            gi.add((int(rng.choice(groups)), int(rng.integers(0, nqb))))
        rows = sorted((0, g, i) for g, i in gi)
    log(f"oracle estimate of {len(rows)} rows ({estimator}, KV heads {groups})")
    if estimator == "pooled":
        ref = oracle.estimate_rows(x.q, x.k, x.theta, rows=rows, keep_margins=False,
                                   block_q=x.block_q, block_k=x.block_k, sink=x.sink,
                                   local=x.local, granularity=x.granularity)
    else:
        ref = oracle.estimate_rows_sale(x.q, x.k, x.theta, rows=rows, keep_margins=False,
                                        block_q=x.block_q, block_k=x.block_k, sink=x.sink,
                                        local=x.local,
                                        lowbit="mxfp4" if estimator == "relative_mxfp4" else "int8")
    nrows, entries, flips = compare_lists(lists, ref)
    log(f"  lists ok: rows={nrows} entries={entries} ambiguous flips={flips}")
    counts = lists.counts.cpu().numpy()
    idx = lists.idx.cpu().numpy()
    same = [key for key, r in ref.items()
            if np.array_equal(idx[key][:counts[key]], r["kept"])]
    pick = [same[j] for j in rng.permutation(len(same))[:n_attn]]
    # always include the last query block of some group (longest lists)
    last = [key for key in same if key[2] == nqb - 1]
    if last and last[0] not in pick:
        pick[-1] = last[0]
    pick.sort()                                  # grouped by KV head for the oracle
    arows = [(b, g * G + int(rng.integers(0, G)), i) for (b, g, i) in pick]
    log(f"oracle attention of {len(arows)} query blocks")
    res = oracle.attention_rows(x.q, x.k, x.v, {key: ref[key]["kept"] for key in pick},
                                rows=arows, block_q=x.block_q, block_k=x.block_k,
                                granularity=x.granularity)
    og, lg = run["o"], run["lse"]
    errs, lerrs = [], []
    for (b, h, i), (oref, lref) in res.items():
        r0 = i * x.block_q
        r1 = min(N, r0 + x.block_q)
        errs.append(np.abs(og[b, r0:r1, h, :].numpy() - oref).ravel())
        lerrs.append(np.abs(lg[b, h, r0:r1] - lref))
    err = np.concatenate(errs)
    lerr = np.concatenate(lerrs)
    log(f"  attention: max|dO|={err.max():.2e} mean={err.mean():.2e} max|dLSE|={lerr.max():.2e}")
    assert err.max() < MAX_ABS and err.mean() < MEAN_ABS and lerr.max() < 1e-2
    assert flips <= max(2, entries // 1000)
    if reuse:
        sref = oracle.anchor_state_rows(x.q, x.k, x.v, block_q=x.block_q, sink=x.sink,
                                        local=x.local, rows=arows)
        so, sl = run["st"]
        e1, e2 = [], []
        for (b, h, i), (oa, la) in sref.items():
            r0 = i * x.block_q
            r1 = min(N, r0 + x.block_q)
            e1.append(np.abs(so[b, r0:r1, h, :] - oa).ravel())
            e2.append(np.abs(sl[b, h, r0:r1] - la))
        e1, e2 = np.concatenate(e1), np.concatenate(e2)
        log(f"  anchor state: max|dO|={e1.max():.2e} mean={e1.mean():.2e} max|dLSE|={e2.max():.2e}")
        assert e1.max() < MAX_ABS and e1.mean() < MEAN_ABS and e2.max() < 1e-2


def test_llama8b_32k_every_row(dev):
    _prefill_parity(dev, "llama8b_32k", n_rows=None, n_attn=16)


def test_llama8b_32k_relative_sampled(dev):
    """SALE's element-wise estimator at the 32K workload (theta 4.0 on every head keeps about
    half of the blocks there)."""
    _prefill_parity(dev, "llama8b_32k", n_rows=32, n_attn=10, estimator="relative")


@pytest.mark.parametrize("g", range(8))
def test_llama8b_128k_every_row(dev, g):
    """The headline workload, one KV head per case (one GPU run for all eight): every (b, g, i)
    list of the 128K layer against the oracle, and the attention of 25 query blocks per KV
    head, 200 in all (random, plus a last block)."""
    _prefill_parity(dev, "llama8b_128k", n_rows=None, n_attn=25, groups=[g])


def test_llama8b_128k_relative_sampled(dev):
    """SALE's element-wise int8 estimator at 128K in bench.py's configuration for it
    (--estimator relative --theta 4.83, i.e. tau = 0.008 on every head)."""
    _prefill_parity(dev, "llama8b_128k", n_rows=16, n_attn=6, estimator="relative", theta=4.83)


def test_llama8b_32k_relative_mxfp4_sampled(dev):
    """The MXFP4 relative estimator at 32K in bench.py's configuration for it
    (--estimator relative_mxfp4 --theta 4.83)."""
    _prefill_parity(dev, "llama8b_32k", n_rows=32, n_attn=10, estimator="relative_mxfp4",
                    theta=4.83)


@pytest.mark.parametrize("name", ["llama8b_32k", "llama8b_128k", "stripe_64k"])
def test_anchor_reuse_sampled(dev, name):
    """Anchor-state reuse in the launch configuration bench.py --anchor-reuse times (block
    lists at 32K and 128K, column lists at 64K)."""
    _prefill_parity(dev, name, n_rows=24, n_attn=10, reuse=True)


@pytest.mark.parametrize("gs", [(0, 1, 2, 3), (4, 5, 6, 7)])
def test_stripe_64k_every_row(dev, gs):
    """Every column list of the 64K stripe workload against the oracle (four KV heads per
    case, one GPU run for both), and the attention of 8 query blocks per case."""
    _prefill_parity(dev, "stripe_64k", n_rows=None, n_attn=8, groups=gs)


@pytest.mark.parametrize("summary", ["bf16", "q4", "fp4", "bf16-topp"])
def test_decode_b16_128k(dev, summary):
    """bf16-topp: top_p = 0.5 with a cap of 256 blocks, which the budgets of this workload
    (about 80 to 200 blocks) stay under."""
    import torch
    import block_sparse_attention_estimate_amd as sa
    log(f"generating decode_b16_128k ({summary} summaries)")
    x = synth.make_decode("decode_b16_128k")
    B, Hq, D = x.q.shape
    q, kc, vc = to_dev(x.q, dev), to_dev(x.k_cache, dev), to_dev(x.v_cache, dev)
    cl = torch.from_numpy(x.cache_len).to(dev)
    kbar = sa.build_block_summary(kc, cl, block_k=x.block_k)
    summ = kbar
    if summary == "q4":
        summ = sa.quantize_block_summary(kbar, block_k=x.block_k)
    elif summary == "fp4":
        summ = sa.quantize_block_summary_fp4(kbar, block_k=x.block_k)
    top_p, top_k = (0.5, 256) if summary == "bf16-topp" else (0.0, x.top_k)
    o, lse, sel = sa.sparse_decode(q, kc, vc, summ, cl, block_k=x.block_k, top_k=top_k,
                                   sink=x.sink, local=x.local, top_p=top_p)
    torch.cuda.synchronize()
    log("oracle block summaries")
    kbar_ref = oracle.block_summary(x.k_cache, x.cache_len, x.block_k)
    kb = kbar.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(kb, kbar_ref)
    score_src = kbar_ref
    if summary == "q4":
        c_ref, s_ref = oracle.quantize_summary_q4(kbar_ref)
        np.testing.assert_array_equal(summ[0].cpu().numpy(), oracle.pack_q4(c_ref))
        np.testing.assert_array_equal(summ[1].view(torch.int16).cpu().numpy().view(np.uint16), s_ref)
        score_src = oracle.dequantize_summary_q4(c_ref, s_ref)
    elif summary == "fp4":
        v_ref, e_ref = oracle.quantize_summary_fp4(kbar_ref)
        c_ref, eb_ref = oracle.pack_fp4(kbar_ref, v_ref, e_ref)
        np.testing.assert_array_equal(summ[0].cpu().numpy(), c_ref)
        np.testing.assert_array_equal(summ[1].cpu().numpy(), eb_ref)
        score_src = oracle.dequantize_summary_fp4(v_ref, e_ref)
    ref = oracle.decode_select(x.q, score_src, x.cache_len, block_k=x.block_k, top_k=top_k,
                               sink=x.sink, local=x.local, top_p=top_p)
    s = sel.cpu().numpy()
    if top_p > 0:
        used, off, flips = check_topp_selection(s, ref)
        budgets = [r["budget"] for r in ref.values()]
        log(f"  top-p selection ok: budgets {min(budgets)}..{max(budgets)} one-off={off} flips={flips}")
        assert max(budgets) < top_k - 5
        O, LSE = oracle.decode_attention(x.q, x.k_cache, x.v_cache, x.cache_len, used,
                                         block_k=x.block_k)
        err = np.abs(o.float().cpu().numpy() - O)
        log(f"  decode attention: max|dO|={err.max():.2e} mean={err.mean():.2e}")
        assert err.max() < MAX_ABS and err.mean() < MEAN_ABS
        assert np.abs(lse.cpu().numpy() - LSE).max() < 1e-2
        return
    flips = 0
    same = {}
    for (b, g), r in ref.items():
        got = s[b, g]
        diff = set(got.tolist()) ^ set(r["selected"].tolist())
        assert diff <= set(r["ambiguous"].tolist()), ((b, g), sorted(diff))
        flips += len(diff)
        if not diff:
            same[(b, g)] = r["selected"]
    log(f"  selection ok: flips={flips}")
    keep_b = [b for b in range(B) if all((b, g) in same for g in range(kc.shape[2]))]
    assert keep_b
    sub = {(j, g): same[(b, g)] for j, b in enumerate(keep_b) for g in range(kc.shape[2])}
    O, LSE = oracle.decode_attention(x.q[keep_b], x.k_cache[keep_b], x.v_cache[keep_b],
                                     x.cache_len[keep_b], sub, block_k=x.block_k)
    err = np.abs(o.float().cpu().numpy()[keep_b] - O)
    log(f"  decode attention over {len(keep_b)} sequences: max|dO|={err.max():.2e} mean={err.mean():.2e}")
    assert err.max() < MAX_ABS and err.mean() < MEAN_ABS
    assert np.abs(lse.cpu().numpy()[keep_b] - LSE).max() < 1e-2
