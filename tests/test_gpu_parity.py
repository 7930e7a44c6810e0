"""GPU parity: the HIP path (through the C ABI) against the oracle on seeded inputs.

Sizes here run in seconds on the oracle yet span several tiles and a ragged tail; the
full-size workloads are in test_gpu_fullsize.py.  Bars: kept lists bit-exact except
entries whose oracle margin lies within 1e-3 of the threshold; attention output under the
oracle's lists within max-abs 2e-2 and mean-abs 2e-3 of the fp64 oracle.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import (MAX_ABS, MEAN_ABS, check_topp_selection, compare_lists, compare_outputs, log,
                     lists_from_ref,
                     oracle_estimate_for, to_dev, upload_lists)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    import block_sparse_attention_estimate_amd as sa
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sa.load_library()
    return torch.device("cuda:0")


def _run_prefill_case(dev, x, theta, *, check_attention=True, stride=None):
    import torch
    import block_sparse_attention_estimate_amd as sa
    B, N, Hq, D = x.q.shape
    Hkv = x.k.shape[2]
    log(f"case {x.name} N={N} Hq={Hq} Hkv={Hkv} d={D} gran={x.granularity} theta={list(np.unique(theta))}")
    q, k, v = to_dev(x.q, dev), to_dev(x.k, dev), to_dev(x.v, dev)
    kw = dict(block_q=x.block_q, block_k=x.block_k, sink=x.sink, local=x.local)
    lists = sa.estimate_mask(q, k, theta, granularity=x.granularity, margins=True, stride=stride,
                             **kw)
    torch.cuda.synchronize()
    ref = oracle_estimate_for(x, theta)
    rows, entries, flips = compare_lists(lists, ref)
    # margins agree with the oracle's within the band on every candidate
    mg = lists.margins.cpu().numpy()
    worst = 0.0
    for (b, g, i), r in ref.items():
        m_ref = r["margin"]
        m_gpu = mg[b, g, i, :m_ref.size]
        fin = np.isfinite(m_ref)
        assert np.array_equal(np.isfinite(m_gpu), fin)
        if fin.any():
            worst = max(worst, float(np.abs(m_gpu[fin] - m_ref[fin]).max()))
    assert worst < 1e-3, worst
    log(f"  lists ok: rows={rows} entries={entries} ambiguous flips={flips} max|dmargin|={worst:.1e}")
    if not check_attention:
        return
    nqb = -(-N // x.block_q)
    st = lists.stride
    dl = upload_lists(ref, (B, Hkv, nqb), dev, x.granularity, st)
    o, lse = sa.sparse_prefill(q, k, v, dl, **kw)
    torch.cuda.synchronize()
    O, LSE = oracle.attention_all(x.q, x.k, x.v, lists_from_ref(ref), block_q=x.block_q,
                                  block_k=x.block_k, granularity=x.granularity)
    mx, mean, lmax = compare_outputs(o, lse, O, LSE)
    log(f"  attention ok: max|dO|={mx:.2e} mean={mean:.2e} max|dLSE|={lmax:.2e}")


def test_tiny_workload_and_theta_sweep(dev):
    x = synth.make_prefill("tiny_4k")
    for th in [4.0, 1.5, 2.0, 2.5, np.inf, -np.inf]:
        _run_prefill_case(dev, x, np.full(1, th, np.float32), check_attention=th in (4.0, 2.5, -np.inf))


@pytest.mark.parametrize("seq,hq,hkv,d,bq", [(4000, 8, 2, 128, 128), (1500, 16, 2, 128, 128),
                                             (1000, 4, 2, 64, 64), (777, 2, 2, 128, 128),
                                             (2100, 4, 1, 64, 128)])
def test_llama_recipe_reduced(dev, seq, hq, hkv, d, bq):
    x = synth.make_prefill("llama8b_32k", seq=seq, hq=hq, hkv=hkv, head_dim=d)
    x.block_q = bq
    grp = hq // hkv
    theta = np.repeat(np.array([2.0, 3.0, 4.0, 6.0] * 8, np.float32)[:hkv], grp)
    _run_prefill_case(dev, x, theta)


def test_edge_lengths(dev):
    for seq in [1, 63, 64, 65, 129, 200]:
        x = synth.make_prefill("llama8b_32k", seq=seq, hq=4, hkv=1)
        _run_prefill_case(dev, x, np.full(4, 3.0, np.float32))


@pytest.mark.parametrize("seq,theta", [(3000, 3.0), (2500, 5.0)])
def test_stripe_reduced(dev, seq, theta):
    x = synth.make_prefill("stripe_64k", seq=seq, hq=8, hkv=2)
    _run_prefill_case(dev, x, np.full(8, theta, np.float32))


@pytest.mark.parametrize("seq,hq,hkv,d,bq", [(1500, 2, 2, 128, 128), (1300, 4, 2, 64, 64),
                                             (1100, 8, 1, 64, 128), (777, 2, 1, 128, 64)])
def test_stripe_shapes(dev, seq, hq, hkv, d, bq):
    """Column lists with 1, 2 and 8 query heads per KV head, head_dim 64 and 128, 64- and
    128-row query blocks (every instance of the gathered-row attention)."""
    x = synth.make_prefill("stripe_64k", seq=seq, hq=hq, hkv=hkv, head_dim=d)
    x.block_q = bq
    grp = hq // hkv
    theta = np.repeat(np.array([3.0, 5.0], np.float32)[:hkv], grp)
    _run_prefill_case(dev, x, theta)


def test_stripe_capacity_overflow_reported(dev):
    import torch
    import block_sparse_attention_estimate_amd as sa
    x = synth.make_prefill("stripe_64k", seq=1000, hq=4, hkv=1)
    q, k = to_dev(x.q, dev), to_dev(x.k, dev)
    lists = sa.estimate_mask(q, k, np.inf, granularity="stripe", stride=300,
                             block_q=128, block_k=64, sink=32, local=256)
    torch.cuda.synchronize()
    counts = lists.counts.cpu().numpy()
    # theta = +inf keeps every causal column: the true counts are reported
    want = [min(1000, (i + 1) * 128) for i in range(counts.shape[2])]
    assert counts[0, 0].tolist() == want
    assert lists.overflowed()
    # the prefill reads only the first `stride` entries of an overflowed row (no fault)
    v = to_dev(x.v, dev)
    o, _ = sa.sparse_prefill(q, k, v, lists, block_q=128, block_k=64, sink=32, local=256)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()


def test_determinism(dev):
    import torch
    import block_sparse_attention_estimate_amd as sa
    x = synth.make_prefill("llama8b_32k", seq=3000, hq=8, hkv=2)
    q, k, v = to_dev(x.q, dev), to_dev(x.k, dev), to_dev(x.v, dev)
    kw = dict(block_q=128, block_k=64, sink=32, local=256)
    outs = []
    for _ in range(2):
        l = sa.estimate_mask(q, k, np.full(8, 6.0, np.float32), **kw)
        o, lse = sa.sparse_prefill(q, k, v, l, **kw)
        torch.cuda.synchronize()
        outs.append((l.counts.cpu(), l.idx.cpu(), o.cpu(), lse.cpu()))
    c0, i0, o0, l0 = outs[0]
    c1, i1, o1, l1 = outs[1]
    assert torch.equal(c0, c1)
    for r in range(c0.numel()):
        n = int(c0.view(-1)[r])
        assert torch.equal(i0.view(-1, i0.shape[-1])[r, :n], i1.view(-1, i1.shape[-1])[r, :n])
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(l0, l1)


@pytest.mark.parametrize("batch,seq,hq,hkv,d,top_k,bk", [(3, 5000, 8, 2, 128, 24, 64),
                                                        (2, 3000, 4, 1, 64, 8, 64),
                                                        (2, 2000, 16, 2, 128, 64, 64),
                                                        (2, 3000, 2, 2, 64, 12, 64),
                                                        (2, 3000, 8, 2, 128, 24, 32),
                                                        (1, 140000, 4, 1, 64, 32, 64)])
def test_decode_reduced(dev, batch, seq, hq, hkv, d, top_k, bk):
    import torch
    import block_sparse_attention_estimate_amd as sa
    x = synth.make_decode(batch=batch, seq=seq, hq=hq, hkv=hkv, head_dim=d, top_k=top_k)
    if batch >= 2:
        x.cache_len[1] = seq - 937          # ragged cache lengths
    log(f"decode B={batch} L={seq} Hq={hq} Hkv={hkv} d={d} K={top_k} bk={bk} lens={x.cache_len.tolist()}")
    q, kc, vc = to_dev(x.q, dev), to_dev(x.k_cache, dev), to_dev(x.v_cache, dev)
    cl = torch.from_numpy(x.cache_len).to(dev)
    kbar = sa.build_block_summary(kc, cl, block_k=bk)
    o, lse, sel = sa.sparse_decode(q, kc, vc, kbar, cl, block_k=bk, top_k=top_k, sink=32, local=256)
    torch.cuda.synchronize()
    kbar_ref = oracle.block_summary(x.k_cache, x.cache_len, bk)
    kb = kbar.view(torch.int16).cpu().numpy().view(np.uint16)
    for b in range(batch):
        nb = -(-int(x.cache_len[b]) // bk)
        np.testing.assert_array_equal(kb[b, :nb], kbar_ref[b, :nb])
    ref = oracle.decode_select(x.q, kbar_ref, x.cache_len, block_k=bk, top_k=top_k, sink=32, local=256)
    s = sel.cpu().numpy()
    used = {}
    flips = 0
    for (b, g), r in ref.items():
        k_ = min(top_k, -(-int(x.cache_len[b]) // bk))
        got = s[b, g, :k_]
        assert (s[b, g, k_:] == -1).all()
        assert np.all(np.diff(got) > 0)
        diff = set(got.tolist()) ^ set(r["selected"].tolist())
        assert diff <= set(r["ambiguous"].tolist()), ((b, g), sorted(diff))
        flips += len(diff)
        used[(b, g)] = got
    O, LSE = oracle.decode_attention(x.q, x.k_cache, x.v_cache, x.cache_len, used, block_k=bk)
    err = np.abs(o.float().cpu().numpy() - O)
    assert err.max() < 2e-2 and err.mean() < 2e-3, (err.max(), err.mean())
    assert np.abs(lse.cpu().numpy() - LSE).max() < 1e-2
    log(f"  decode ok: flips={flips} max|dO|={err.max():.2e} mean={err.mean():.2e}")


@pytest.mark.parametrize("batch,seq,hq,hkv,d,top_k,bk", [(3, 5000, 8, 2, 128, 24, 64), (2, 3000, 4, 1, 64, 8, 64),
                                                        (2, 3000, 4, 4, 128, 12, 64),    # G = 1
                                                        (3, 2500, 8, 4, 64, 16, 64),     # G = 2
                                                        (2, 2100, 8, 2, 128, 20, 32)])   # 32-key blocks
def test_decode_q4_reduced(dev, batch, seq, hq, hkv, d, top_k, bk):
    """4-bit summaries: codes and scales bit-exact, selection from scale * code within the
    ambiguity band, attention over the selection as for bf16 summaries; groups of 1, 2 and 4
    query heads and 32-key blocks."""
    import torch
    import block_sparse_attention_estimate_amd as sa
    x = synth.make_decode(batch=batch, seq=seq, hq=hq, hkv=hkv, head_dim=d, top_k=top_k)
    if batch >= 2:
        x.cache_len[1] = seq - 937
    log(f"decode q4 B={batch} L={seq} Hq={hq} Hkv={hkv} d={d} K={top_k} bk={bk}")
    q, kc, vc = to_dev(x.q, dev), to_dev(x.k_cache, dev), to_dev(x.v_cache, dev)
    cl = torch.from_numpy(x.cache_len).to(dev)
    kbar = sa.build_block_summary(kc, cl, block_k=bk)
    codes, scales = sa.quantize_block_summary(kbar, block_k=bk)
    o, lse, sel = sa.sparse_decode(q, kc, vc, (codes, scales), cl, block_k=bk, top_k=top_k,
                                   sink=32, local=256)
    torch.cuda.synchronize()
    kbar_ref = oracle.block_summary(x.k_cache, x.cache_len, bk)
    c_ref, s_ref = oracle.quantize_summary_q4(kbar_ref)
    np.testing.assert_array_equal(codes.cpu().numpy(), oracle.pack_q4(c_ref))
    np.testing.assert_array_equal(scales.view(torch.int16).cpu().numpy().view(np.uint16), s_ref)
    deq = oracle.dequantize_summary_q4(c_ref, s_ref)
    ref = oracle.decode_select(x.q, deq, x.cache_len, block_k=bk, top_k=top_k, sink=32, local=256)
    s = sel.cpu().numpy()
    used, flips = {}, 0
    for (b, g), r in ref.items():
        k_ = min(top_k, -(-int(x.cache_len[b]) // bk))
        got = s[b, g, :k_]
        assert (s[b, g, k_:] == -1).all() and np.all(np.diff(got) > 0)
        diff = set(got.tolist()) ^ set(r["selected"].tolist())
        assert diff <= set(r["ambiguous"].tolist()), ((b, g), sorted(diff))
        flips += len(diff)
        used[(b, g)] = got
    O, LSE = oracle.decode_attention(x.q, x.k_cache, x.v_cache, x.cache_len, used, block_k=bk)
    err = np.abs(o.float().cpu().numpy() - O)
    assert err.max() < 2e-2 and err.mean() < 2e-3, (err.max(), err.mean())
    assert np.abs(lse.cpu().numpy() - LSE).max() < 1e-2
    log(f"  decode q4 ok: flips={flips} max|dO|={err.max():.2e}")


@pytest.mark.parametrize("batch,seq,hq,hkv,d,top_k,bk", [(3, 5000, 8, 2, 128, 24, 64), (2, 3000, 4, 1, 64, 8, 64),
                                                        (2, 1000, 16, 2, 128, 6, 64),
                                                        (2, 3000, 4, 4, 128, 12, 64),    # G = 1
                                                        (3, 2500, 8, 4, 64, 16, 64),     # G = 2
                                                        (2, 2100, 8, 2, 128, 20, 32),    # 32-key blocks
                                                        (2, 1300, 2, 2, 128, 10, 32)])   # G = 1, bk 32, K = |F| max
def test_decode_fp4_reduced(dev, batch, seq, hq, hkv, d, top_k, bk):
    """FP4 (MXFP4) summaries: codes and exponents bit-exact, selection from the E2M1 values
    times 2^e within the ambiguity band, attention over the selection as for bf16 summaries.
    Groups of 1, 2, 4 and 8 query heads (the scorer puts the group's heads on MFMA rows, so
    small groups leave most rows empty) and 32-key blocks."""
    import torch
    import block_sparse_attention_estimate_amd as sa
    x = synth.make_decode(batch=batch, seq=seq, hq=hq, hkv=hkv, head_dim=d, top_k=top_k)
    if batch >= 2:
        x.cache_len[1] = seq - 937
    log(f"decode fp4 B={batch} L={seq} Hq={hq} Hkv={hkv} d={d} K={top_k} bk={bk}")
    q, kc, vc = to_dev(x.q, dev), to_dev(x.k_cache, dev), to_dev(x.v_cache, dev)
    cl = torch.from_numpy(x.cache_len).to(dev)
    kbar = sa.build_block_summary(kc, cl, block_k=bk)
    codes, exps = sa.quantize_block_summary_fp4(kbar, block_k=bk)
    o, lse, sel = sa.sparse_decode(q, kc, vc, (codes, exps), cl, block_k=bk, top_k=top_k,
                                   sink=32, local=256)
    torch.cuda.synchronize()
    kbar_ref = oracle.block_summary(x.k_cache, x.cache_len, bk)
    v_ref, e_ref = oracle.quantize_summary_fp4(kbar_ref)
    c_ref, eb_ref = oracle.pack_fp4(kbar_ref, v_ref, e_ref)
    np.testing.assert_array_equal(codes.cpu().numpy(), c_ref)
    np.testing.assert_array_equal(exps.cpu().numpy(), eb_ref)
    deq = oracle.dequantize_summary_fp4(v_ref, e_ref)
    ref = oracle.decode_select(x.q, deq, x.cache_len, block_k=bk, top_k=top_k, sink=32, local=256)
    s = sel.cpu().numpy()
    used, flips = {}, 0
    for (b, g), r in ref.items():
        k_ = min(top_k, -(-int(x.cache_len[b]) // bk))
        got = s[b, g, :k_]
        assert (s[b, g, k_:] == -1).all() and np.all(np.diff(got) > 0)
        diff = set(got.tolist()) ^ set(r["selected"].tolist())
        assert diff <= set(r["ambiguous"].tolist()), ((b, g), sorted(diff))
        flips += len(diff)
        used[(b, g)] = got
    O, LSE = oracle.decode_attention(x.q, x.k_cache, x.v_cache, x.cache_len, used, block_k=bk)
    err = np.abs(o.float().cpu().numpy() - O)
    assert err.max() < 2e-2 and err.mean() < 2e-3, (err.max(), err.mean())
    assert np.abs(lse.cpu().numpy() - LSE).max() < 1e-2
    log(f"  decode fp4 ok: flips={flips} max|dO|={err.max():.2e}")


@pytest.mark.parametrize("batch,seq,hq,hkv,d,top_k,bk,top_p,summary",
                         [(3, 5000, 8, 2, 128, 79, 64, 0.5, "bf16"),
                          (2, 3000, 4, 1, 64, 47, 64, 0.9, "bf16"),
                          (2, 3000, 8, 2, 128, 12, 64, 0.9, "bf16"),    # the cap of K binds
                          (2, 3000, 8, 2, 128, 94, 32, 0.7, "bf16"),
                          (2, 5000, 8, 2, 128, 79, 64, 0.02, "bf16"),   # forced share suffices
                          (3, 5000, 8, 2, 128, 79, 64, 0.8, "q4"),
                          (2, 3000, 4, 1, 64, 47, 64, 0.8, "fp4")])
def test_decode_topp_reduced(dev, batch, seq, hq, hkv, d, top_k, bk, top_p, summary):
    """Top-p budget: per (b, g) the forced blocks plus the oracle's budget of content blocks
    (one off only where the oracle's cumulative share lies within its band of top_p), in the
    oracle's score order outside the score band; attention over the GPU's selection."""
    import torch
    import block_sparse_attention_estimate_amd as sa
    x = synth.make_decode(batch=batch, seq=seq, hq=hq, hkv=hkv, head_dim=d, top_k=top_k)
    if batch >= 2:
        x.cache_len[1] = seq - 937
    log(f"decode top-p={top_p} {summary} B={batch} L={seq} Hq={hq} Hkv={hkv} d={d} K={top_k} bk={bk}")
    q, kc, vc = to_dev(x.q, dev), to_dev(x.k_cache, dev), to_dev(x.v_cache, dev)
    cl = torch.from_numpy(x.cache_len).to(dev)
    kbar = sa.build_block_summary(kc, cl, block_k=bk)
    summ = kbar
    if summary == "q4":
        summ = sa.quantize_block_summary(kbar, block_k=bk)
    elif summary == "fp4":
        summ = sa.quantize_block_summary_fp4(kbar, block_k=bk)
    o, lse, sel = sa.sparse_decode(q, kc, vc, summ, cl, block_k=bk, top_k=top_k, sink=32,
                                   local=256, top_p=top_p)
    torch.cuda.synchronize()
    kbar_ref = oracle.block_summary(x.k_cache, x.cache_len, bk)
    if summary == "q4":
        kbar_ref = oracle.dequantize_summary_q4(*oracle.quantize_summary_q4(kbar_ref))
    elif summary == "fp4":
        kbar_ref = oracle.dequantize_summary_fp4(*oracle.quantize_summary_fp4(kbar_ref))
    ref = oracle.decode_select(x.q, kbar_ref, x.cache_len, block_k=bk, top_k=top_k, sink=32,
                               local=256, top_p=top_p)
    used, off, flips = check_topp_selection(sel.cpu().numpy(), ref)
    budgets = [r["budget"] for r in ref.values()]
    O, LSE = oracle.decode_attention(x.q, x.k_cache, x.v_cache, x.cache_len, used, block_k=bk)
    err = np.abs(o.float().cpu().numpy() - O)
    assert err.max() < 2e-2 and err.mean() < 2e-3, (err.max(), err.mean())
    assert np.abs(lse.cpu().numpy() - LSE).max() < 1e-2
    log(f"  top-p ok: budgets {min(budgets)}..{max(budgets)} one-off={off} flips={flips} "
        f"max|dO|={err.max():.2e}")


@pytest.mark.parametrize("estimator", ["relative", "relative_mxfp4"])
@pytest.mark.parametrize("seq,hq,hkv,d,bq", [(4000, 8, 2, 128, 128), (1500, 16, 2, 128, 128),
                                             (1000, 4, 2, 64, 64), (777, 2, 2, 128, 128),
                                             (2100, 4, 1, 64, 128), (200, 4, 1, 128, 64)])
def test_relative_estimator_reduced(dev, seq, hq, hkv, d, bq, estimator):
    """SALE's element-wise estimate (int8 or MXFP4 operands): lists bit-exact outside the band,
    margins within 1e-3 of the oracle's, at thetas from forced-only to dense; attention under
    the oracle's lists."""
    lowbit = "mxfp4" if estimator == "relative_mxfp4" else "int8"
    import torch
    import block_sparse_attention_estimate_amd as sa
    x = synth.make_prefill("llama8b_32k", seq=seq, hq=hq, hkv=hkv, head_dim=d)
    x.block_q = bq
    grp = hq // hkv
    q, k, v = to_dev(x.q, dev), to_dev(x.k, dev), to_dev(x.v, dev)
    kw = dict(block_q=bq, block_k=64, sink=32, local=256)
    base = np.repeat(np.array([4.0, 6.0, 8.0, 5.0] * 8, np.float32)[:hkv], grp)
    for theta in [base, np.full(hq, -np.inf, np.float32), np.full(hq, np.inf, np.float32),
                  base + np.linspace(0, 1, hq, dtype=np.float32)]:
        log(f"{estimator} N={seq} Hq={hq} Hkv={hkv} d={d} bq={bq} theta={np.unique(theta)[:4]}")
        lists = sa.estimate_mask(q, k, theta, estimator=estimator, margins=True, **kw)
        torch.cuda.synchronize()
        ref = oracle.estimate_all_sale(x.q, x.k, theta, lowbit=lowbit, **kw)
        rows, entries, flips = compare_lists(lists, ref)
        mg = lists.margins.cpu().numpy()
        worst = 0.0
        for (b, g, i), r in ref.items():
            m_ref = r["margin"]
            m_gpu = mg[b, g, i, :m_ref.size]
            fin = np.isfinite(m_ref)
            assert np.array_equal(np.isfinite(m_gpu), fin), (b, g, i)
            if fin.any():
                worst = max(worst, float(np.abs(m_gpu[fin] - m_ref[fin]).max()))
        assert worst < 1e-3, worst
        log(f"  lists ok: entries={entries} flips={flips} max|dmargin|={worst:.1e}")
    nqb = -(-seq // bq)
    dl = upload_lists(ref, (1, hkv, nqb), dev, "block", lists.stride)
    o, lse = sa.sparse_prefill(q, k, v, dl, **kw)
    torch.cuda.synchronize()
    O, LSE = oracle.attention_all(x.q, x.k, x.v, lists_from_ref(ref), block_q=bq, block_k=64,
                                  granularity="block")
    compare_outputs(o, lse, O, LSE)


@pytest.mark.parametrize("name,seq,estimator,step", [("llama8b_32k", 4000, "pooled", 4),
                                                    ("llama8b_32k", 4000, "pooled", 16),
                                                    ("stripe_64k", 3000, "pooled", 4),
                                                    ("llama8b_32k", 3000, "relative", 16),
                                                    ("llama8b_32k", 2100, "relative", 3)])
def test_step_grouping(dev, name, seq, estimator, step):
    """Grouped identification: lists equal the oracle's grouped lists (bit-exact outside the
    band of any block of the group)."""
    import torch
    import block_sparse_attention_estimate_amd as sa
    x = synth.make_prefill(name, seq=seq, hq=8, hkv=2)
    # thetas at which both estimators select blocks beyond the forced ones on this data
    theta = np.repeat(np.array([11.0, 12.0] if estimator == "pooled" else [4.0, 6.0],
                               np.float32), 4)
    q, k = to_dev(x.q, dev), to_dev(x.k, dev)
    kw = dict(block_q=x.block_q, block_k=x.block_k, sink=x.sink, local=x.local)
    log(f"step={step} {estimator} {name} N={seq}")
    lists = sa.estimate_mask(q, k, theta, granularity=x.granularity, estimator=estimator,
                             step=step, stride=seq if x.granularity == "stripe" else None, **kw)
    torch.cuda.synchronize()
    if estimator == "pooled":
        ref = oracle.estimate_all(x.q, x.k, theta, granularity=x.granularity, **kw)
    else:
        ref = oracle.estimate_all_sale(x.q, x.k, theta, **kw)
    grouped = oracle.group_step(ref, step)
    rows, entries, flips = compare_lists(lists, grouped)
    plain = sum(r["kept"].size for r in ref.values())
    log(f"  grouped lists ok: entries={entries} (ungrouped {plain}) flips={flips}")
    assert entries > plain


@pytest.mark.parametrize("top_p,top_k", [(0.0, 64), (0.5, 8192)])
def test_decode_max_cache(dev, top_p, top_k):
    """The largest cache the library takes: 8192 blocks of 64 keys (524288 tokens), fixed K
    and a top-p budget over every block."""
    import torch
    import block_sparse_attention_estimate_amd as sa
    L = 8192 * 64
    x = synth.make_decode(batch=1, seq=L, hq=4, hkv=1, head_dim=64, top_k=top_k)
    log(f"decode max cache L={L} top_p={top_p} K={top_k}")
    q, kc, vc = to_dev(x.q, dev), to_dev(x.k_cache, dev), to_dev(x.v_cache, dev)
    cl = torch.from_numpy(x.cache_len).to(dev)
    kbar = sa.build_block_summary(kc, cl, block_k=64)
    o, lse, sel = sa.sparse_decode(q, kc, vc, kbar, cl, block_k=64, top_k=top_k, sink=32,
                                   local=256, top_p=top_p)
    torch.cuda.synchronize()
    kbar_ref = oracle.block_summary(x.k_cache, x.cache_len, 64)
    np.testing.assert_array_equal(kbar.view(torch.int16).cpu().numpy().view(np.uint16), kbar_ref)
    ref = oracle.decode_select(x.q, kbar_ref, x.cache_len, block_k=64, top_k=top_k, sink=32,
                               local=256, top_p=top_p)
    s = sel.cpu().numpy()
    if top_p > 0:
        used, off, flips = check_topp_selection(s, ref)
        log(f"  budget {ref[(0, 0)]['budget']} one-off={off} flips={flips}")
    else:
        used, flips = {}, 0
        for (b, g), r in ref.items():
            got = s[b, g]
            assert np.all(np.diff(got) > 0)
            diff = set(got.tolist()) ^ set(r["selected"].tolist())
            assert diff <= set(r["ambiguous"].tolist()), sorted(diff)
            flips += len(diff)
            used[(b, g)] = got
    O, LSE = oracle.decode_attention(x.q, x.k_cache, x.v_cache, x.cache_len, used, block_k=64)
    err = np.abs(o.float().cpu().numpy() - O)
    assert err.max() < 2e-2 and err.mean() < 2e-3, (err.max(), err.mean())
    assert np.abs(lse.cpu().numpy() - LSE).max() < 1e-2


@pytest.mark.parametrize("name,estimator", [("llama8b_32k", "pooled"), ("stripe_64k", "pooled"),
                                            ("llama8b_32k", "relative"),
                                            ("llama8b_32k", "relative_mxfp4")])
def test_batched_prefill(dev, name, estimator):
    """Batch 3 with a ragged length: every batch entry's lists and attention against the
    oracle (the batch strides of every estimate and attention kernel)."""
    import torch
    import block_sparse_attention_estimate_amd as sa
    x = synth.make_prefill(name, seq=2100, batch=3, hq=8, hkv=2)
    theta = np.repeat(np.array([6.0, 11.0] if estimator == "pooled" else [4.0, 6.0],
                               np.float32), 4)
    log(f"batched {name} {estimator} B=3 N=2100")
    q, k, v = to_dev(x.q, dev), to_dev(x.k, dev), to_dev(x.v, dev)
    kw = dict(block_q=x.block_q, block_k=x.block_k, sink=x.sink, local=x.local)
    lists = sa.estimate_mask(q, k, theta, granularity=x.granularity, estimator=estimator,
                             **kw)
    torch.cuda.synchronize()
    if estimator == "pooled":
        ref = oracle.estimate_all(x.q, x.k, theta, granularity=x.granularity, **kw)
    else:
        ref = oracle.estimate_all_sale(x.q, x.k, theta, lowbit="mxfp4" if "mxfp4" in estimator
                                       else "int8", **kw)
    rows, entries, flips = compare_lists(lists, ref)
    assert {b for (b, _, _) in ref} == {0, 1, 2}
    nqb = -(-2100 // x.block_q)
    dl = upload_lists(ref, (3, 2, nqb), dev, x.granularity, lists.stride)
    o, lse = sa.sparse_prefill(q, k, v, dl, **kw)
    torch.cuda.synchronize()
    O, LSE = oracle.attention_all(x.q, x.k, x.v, lists_from_ref(ref), block_q=x.block_q,
                                  block_k=x.block_k, granularity=x.granularity)
    mx, mean, lmax = compare_outputs(o, lse, O, LSE)
    log(f"  batched ok: entries={entries} flips={flips} max|dO|={mx:.2e}")


def _packed(dev, *parts):
    """Tensors [B, N, H_i, d] as views into one [B, N, sum H_i, d] buffer (strided heads)."""
    import torch
    full = torch.cat([to_dev(p, dev) for p in parts], dim=2)
    out, h0 = [], 0
    for p in parts:
        out.append(full[:, :, h0:h0 + p.shape[2]])
        h0 += p.shape[2]
    return out


@pytest.mark.parametrize("granularity", ["block", "stripe"])
def test_packed_qkv_bit_identical(dev, granularity):
    """Q, K and V as head slices of one packed buffer (row strides of (Hq + 2 Hkv) d): lists,
    margins, output and LSE bit-identical to the contiguous tensors."""
    import torch
    import block_sparse_attention_estimate_amd as sa
    name = "llama8b_32k" if granularity == "block" else "stripe_64k"
    x = synth.make_prefill(name, seq=3000, batch=2, hq=8, hkv=2)
    theta = np.repeat(np.array([4.0, 11.0], np.float32), 4)
    kw = dict(block_q=x.block_q, block_k=x.block_k, sink=x.sink, local=x.local)
    res = []
    for packed in (False, True):
        if packed:
            q, k, v = _packed(dev, x.q, x.k, x.v)
            assert not q.is_contiguous()
        else:
            q, k, v = to_dev(x.q, dev), to_dev(x.k, dev), to_dev(x.v, dev)
        lists = sa.estimate_mask(q, k, theta, granularity=granularity, margins=True, **kw)
        o, lse = sa.sparse_prefill(q, k, v, lists, **kw)
        torch.cuda.synchronize()
        res.append((lists.counts.cpu(), lists.idx.cpu(), lists.margins.cpu(), o.cpu(), lse.cpu()))
    (c0, i0, m0, o0, l0), (c1, i1, m1, o1, l1) = res
    assert torch.equal(c0, c1)
    for r in range(c0.numel()):
        n = int(c0.view(-1)[r])
        assert torch.equal(i0.view(-1, i0.shape[-1])[r, :n], i1.view(-1, i1.shape[-1])[r, :n])
    assert torch.equal(torch.nan_to_num(m0, nan=7.0), torch.nan_to_num(m1, nan=7.0))
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)) and torch.equal(l0, l1)


def test_softmax_scale_prefill(dev):
    """A softmax scale other than 1/sqrt(d), against the oracle (estimate and attention)."""
    import torch
    import block_sparse_attention_estimate_amd as sa
    x = synth.make_prefill("llama8b_32k", seq=2100, hq=8, hkv=2)
    scale = 0.05
    theta = np.repeat(np.array([2.0, 3.0], np.float32), 4)
    kw = dict(block_q=x.block_q, block_k=x.block_k, sink=x.sink, local=x.local)
    q, k, v = to_dev(x.q, dev), to_dev(x.k, dev), to_dev(x.v, dev)
    lists = sa.estimate_mask(q, k, theta, softmax_scale=scale, **kw)
    torch.cuda.synchronize()
    ref = oracle.estimate_all(x.q, x.k, theta, scale=scale, **kw)
    rows, entries, flips = compare_lists(lists, ref)
    dl = upload_lists(ref, (1, 2, -(-2100 // x.block_q)), dev, "block", lists.stride)
    o, lse = sa.sparse_prefill(q, k, v, dl, softmax_scale=scale, **kw)
    torch.cuda.synchronize()
    O, LSE = oracle.attention_all(x.q, x.k, x.v, lists_from_ref(ref), block_q=x.block_q,
                                  block_k=x.block_k, scale=scale)
    compare_outputs(o, lse, O, LSE)
    ref_rel = oracle.estimate_all_sale(x.q, x.k, theta + 2.0, scale=scale, **kw)
    lr = sa.estimate_mask(q, k, theta + 2.0, softmax_scale=scale, estimator="relative", **kw)
    torch.cuda.synchronize()
    compare_lists(lr, ref_rel)


def test_decode_packed_cache_and_scale(dev):
    """A K/V cache packed as [B, L, 2 Hkv, d] (strided heads) gives bit-identical decode
    results; a custom softmax scale matches the oracle."""
    import torch
    import block_sparse_attention_estimate_amd as sa
    x = synth.make_decode(batch=2, seq=5000, hq=8, hkv=2, head_dim=128, top_k=24)
    x.cache_len[1] = 4000
    q = to_dev(x.q, dev)
    cl = torch.from_numpy(x.cache_len).to(dev)
    outs = []
    for packed in (False, True):
        if packed:
            kc, vc = _packed(dev, x.k_cache, x.v_cache)
        else:
            kc, vc = to_dev(x.k_cache, dev), to_dev(x.v_cache, dev)
        kbar = sa.build_block_summary(kc, cl, block_k=64)
        o, lse, sel = sa.sparse_decode(q, kc, vc, kbar, cl, block_k=64, top_k=24, sink=32,
                                       local=256, softmax_scale=0.07)
        torch.cuda.synchronize()
        outs.append((kbar.cpu(), o.cpu(), lse.cpu(), sel.cpu()))
    for a_, b_ in zip(*outs):
        assert torch.equal(a_.view(torch.int16) if a_.dtype == torch.bfloat16 else a_,
                           b_.view(torch.int16) if b_.dtype == torch.bfloat16 else b_)
    kbar_ref = oracle.block_summary(x.k_cache, x.cache_len, 64)
    ref = oracle.decode_select(x.q, kbar_ref, x.cache_len, block_k=64, top_k=24, sink=32,
                               local=256, scale=0.07)
    s = outs[1][3].numpy()
    used = {}
    for (b, g), r in ref.items():
        k_ = min(24, -(-int(x.cache_len[b]) // 64))
        got = s[b, g, :k_]
        diff = set(got.tolist()) ^ set(r["selected"].tolist())
        assert diff <= set(r["ambiguous"].tolist()), ((b, g), sorted(diff))
        used[(b, g)] = got
    O, LSE = oracle.decode_attention(x.q, x.k_cache, x.v_cache, x.cache_len, used, block_k=64,
                                     scale=0.07)
    err = np.abs(outs[1][1].float().numpy() - O)
    assert err.max() < 2e-2 and err.mean() < 2e-3, (err.max(), err.mean())
    assert np.abs(outs[1][2].numpy() - LSE).max() < 1e-2


@pytest.mark.parametrize("seq,hq,hkv,d,bq,sink,local", [
    (3000, 8, 2, 128, 128, 32, 256),     # the workloads' sink and window, ragged tail
    (1000, 4, 2, 64, 64, 32, 256),
    (777, 2, 2, 128, 128, 100, 64),      # sink past one key block, window under one block
    (1500, 8, 1, 128, 128, 0, 300),      # no sink; 8 heads per KV head (two rounds per block)
    (900, 4, 1, 64, 128, 5, 600),        # regions of up to 800 rows (four staged chunks)
    (65, 4, 1, 128, 128, 32, 256),       # one query block, ragged
])
def test_anchor_state_reduced(dev, seq, hq, hkv, d, bq, sink, local):
    """Anchor-state reuse: the estimate with the state gives the plain estimate's lists bit for
    bit, the state matches the oracle's attention over each row's anchor region, and the
    resuming prefill under the oracle's lists matches attention over those lists."""
    import torch
    import block_sparse_attention_estimate_amd as sa
    x = synth.make_prefill("llama8b_32k", seq=seq, hq=hq, hkv=hkv, head_dim=d)
    x.block_q, x.sink, x.local = bq, sink, local
    B, N, Hq, D = x.q.shape
    grp = hq // hkv
    theta = np.repeat(np.array([2.0, 3.0, 4.0, 6.0] * 8, np.float32)[:hkv], grp)
    log(f"anchor state N={N} Hq={Hq} Hkv={hkv} d={D} bq={bq} sink={sink} local={local}")
    q, k, v = to_dev(x.q, dev), to_dev(x.k, dev), to_dev(x.v, dev)
    kw = dict(block_q=bq, block_k=64, sink=sink, local=local)
    plain = sa.estimate_mask(q, k, theta, **kw)
    lists, st = sa.estimate_mask_anchor_state(q, k, v, theta, **kw)
    torch.cuda.synchronize()
    assert torch.equal(plain.counts, lists.counts)
    c = plain.counts.cpu().numpy().reshape(-1)
    i0 = plain.idx.cpu().numpy().reshape(c.size, -1)
    i1 = lists.idx.cpu().numpy().reshape(c.size, -1)
    for r in range(c.size):
        assert np.array_equal(i0[r, :c[r]], i1[r, :c[r]])
    ref = oracle_estimate_for(x, theta)
    rows_l, entries, flips = compare_lists(lists, ref)
    nqb = -(-N // bq)
    rows = [(0, h, i) for h in range(Hq) for i in range(nqb)]
    sref = oracle.anchor_state_rows(x.q, x.k, x.v, block_q=bq, sink=sink, local=local, rows=rows)
    so = st.o.float().cpu().numpy()
    sl = st.lse.cpu().numpy()
    errs, lerrs = [], []
    for (b, h, i), (oa, la) in sref.items():
        r0, r1 = i * bq, min(N, (i + 1) * bq)
        errs.append(np.abs(so[b, r0:r1, h, :] - oa).ravel())
        lerrs.append(np.abs(sl[b, h, r0:r1] - la))
    err, lerr = np.concatenate(errs), np.concatenate(lerrs)
    log(f"  lists equal the plain estimate ({rows_l} rows, {flips} ambiguous flips vs oracle); "
        f"state max|dO|={err.max():.2e} mean={err.mean():.2e} max|dLSE|={lerr.max():.2e}")
    assert err.max() < MAX_ABS and err.mean() < MEAN_ABS and lerr.max() < 1e-2
    dl = upload_lists(ref, (B, hkv, nqb), dev, "block", lists.stride)
    o, lse = sa.sparse_prefill_resume(q, k, v, dl, st, **kw)
    torch.cuda.synchronize()
    O, LSE = oracle.attention_all(x.q, x.k, x.v, lists_from_ref(ref), block_q=bq, block_k=64)
    mx, mean, lmax = compare_outputs(o, lse, O, LSE)
    log(f"  resumed attention ok: max|dO|={mx:.2e} mean={mean:.2e} max|dLSE|={lmax:.2e}")


def test_anchor_state_resume_without_rest(dev):
    """Lists of only the forced blocks with local >= N and no sink: every listed causal token is
    in the anchor region, so the resumed prefill returns the state itself."""
    import torch
    import block_sparse_attention_estimate_amd as sa
    x = synth.make_prefill("llama8b_32k", seq=700, hq=4, hkv=1, head_dim=128)
    N = 700
    kw = dict(block_q=128, block_k=64, sink=0, local=N)
    q, k, v = to_dev(x.q, dev), to_dev(x.k, dev), to_dev(x.v, dev)
    lists, st = sa.estimate_mask_anchor_state(q, k, v, -np.inf, **kw)
    o, lse = sa.sparse_prefill_resume(q, k, v, lists, st, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), st.o.view(torch.int16))
    assert torch.allclose(lse, st.lse, rtol=0, atol=1e-5)
    # and the state is dense causal attention here
    O, LSE = oracle.attention_all(x.q, x.k, x.v, {(0, 0, i): np.arange(-(-min(N, (i + 1) * 128) // 64))
                                                  for i in range(-(-N // 128))},
                                  block_q=128, block_k=64)
    mx, mean, lmax = compare_outputs(o, lse, O, LSE)
    log(f"  state = dense causal attention: max|dO|={mx:.2e} mean={mean:.2e} max|dLSE|={lmax:.2e}")


def test_anchor_state_batched_packed_scale(dev):
    """Anchor-state reuse with batch 3, a ragged length, Q/K/V as head slices of one packed
    buffer and a custom softmax scale: state and resumed output against the oracle, and both
    bit-identical to the run on contiguous tensors."""
    import torch
    import block_sparse_attention_estimate_amd as sa
    x = synth.make_prefill("llama8b_32k", seq=2100, batch=3, hq=8, hkv=2)
    N, Hq = 2100, 8
    theta = np.repeat(np.array([6.0, 11.0], np.float32), 4)
    scale = 0.07
    kw = dict(block_q=x.block_q, block_k=x.block_k, sink=x.sink, local=x.local,
              softmax_scale=scale)
    log("anchor state B=3 N=2100 packed, scale 0.07")
    res = []
    for packed in (False, True):
        if packed:
            q, k, v = _packed(dev, x.q, x.k, x.v)
            assert not q.is_contiguous()
        else:
            q, k, v = to_dev(x.q, dev), to_dev(x.k, dev), to_dev(x.v, dev)
        lists, st = sa.estimate_mask_anchor_state(q, k, v, theta, **kw)
        o, lse = sa.sparse_prefill_resume(q, k, v, lists, st, **kw)
        torch.cuda.synchronize()
        res.append((lists, st, o, lse))
    (l0, s0, o0, e0), (l1, s1, o1, e1) = res
    assert torch.equal(l0.counts, l1.counts)
    assert torch.equal(s0.o.view(torch.int16), s1.o.view(torch.int16)) and torch.equal(s0.lse, s1.lse)
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)) and torch.equal(e0, e1)
    ekw = {key: val for key, val in kw.items() if key != "softmax_scale"}
    ref = oracle.estimate_all(x.q, x.k, theta, granularity="block", scale=scale, **ekw)
    compare_lists(l0, ref)
    nqb = -(-N // x.block_q)
    rows = [(b, h, i) for b in range(3) for h in range(Hq) for i in range(nqb)]
    sref = oracle.anchor_state_rows(x.q, x.k, x.v, block_q=x.block_q, sink=x.sink, local=x.local,
                                    rows=rows, scale=scale)
    so, sl = s0.o.float().cpu().numpy(), s0.lse.cpu().numpy()
    err = max(float(np.abs(so[b, i * 128:min(N, i * 128 + 128), h, :] - oa).max())
              for (b, h, i), (oa, la) in sref.items())
    lerr = max(float(np.abs(sl[b, h, i * 128:min(N, i * 128 + 128)] - la).max())
               for (b, h, i), (oa, la) in sref.items())
    assert err < MAX_ABS and lerr < 1e-2
    # resumed output (the GPU's lists, which match the oracle's outside the band) vs the plain
    # definition over those lists
    counts = l0.counts.cpu().numpy()
    idx = l0.idx.cpu().numpy()
    glists = {(b, g, i): idx[b, g, i, :counts[b, g, i]] for b in range(3) for g in range(2)
              for i in range(nqb)}
    O, LSE = oracle.attention_all(x.q, x.k, x.v, glists, block_q=x.block_q, block_k=x.block_k,
                                  scale=scale)
    mx, mean, lmax = compare_outputs(o0, e0, O, LSE)
    log(f"  state max|dO|={err:.2e}; resumed max|dO|={mx:.2e} mean={mean:.2e} max|dLSE|={lmax:.2e}")


@pytest.mark.parametrize("mode", ["stripe", "relative", "relative_mxfp4", "anchor_state"])
def test_determinism_other_paths(dev, mode):
    """Two runs of the same call give bit-identical lists, outputs and LSE (no atomics or
    reduction orders that depend on scheduling)."""
    import torch
    import block_sparse_attention_estimate_amd as sa
    name = "stripe_64k" if mode == "stripe" else "llama8b_32k"
    x = synth.make_prefill(name, seq=3000, hq=8, hkv=2)
    q, k, v = to_dev(x.q, dev), to_dev(x.k, dev), to_dev(x.v, dev)
    kw = dict(block_q=128, block_k=64, sink=32, local=256)
    theta = np.full(8, 5.0 if mode.startswith("relative") else 6.0, np.float32)
    outs = []
    for _ in range(2):
        if mode == "anchor_state":
            lists, st = sa.estimate_mask_anchor_state(q, k, v, theta, **kw)
            o, lse = sa.sparse_prefill_resume(q, k, v, lists, st, **kw)
        else:
            est = mode if mode.startswith("relative") else "pooled"
            gran = "stripe" if mode == "stripe" else "block"
            lists = sa.estimate_mask(q, k, theta, granularity=gran, estimator=est, **kw)
            o, lse = sa.sparse_prefill(q, k, v, lists, **kw)
        torch.cuda.synchronize()
        outs.append((lists.counts.cpu(), lists.idx.cpu(), o.cpu(), lse.cpu()))
    (c0, i0, o0, l0), (c1, i1, o1, l1) = outs
    assert torch.equal(c0, c1)
    for r in range(c0.numel()):
        n = min(int(c0.view(-1)[r]), i0.shape[-1])
        assert torch.equal(i0.view(-1, i0.shape[-1])[r, :n], i1.view(-1, i1.shape[-1])[r, :n])
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(l0, l1)


@pytest.mark.parametrize("top_p", [0.0, 0.5])
def test_decode_determinism(dev, top_p):
    import torch
    import block_sparse_attention_estimate_amd as sa
    x = synth.make_decode("decode_b16_128k", batch=3, seq=5000, hq=8, hkv=2)
    q, kc, vc = to_dev(x.q, dev), to_dev(x.k_cache, dev), to_dev(x.v_cache, dev)
    cl = torch.from_numpy(x.cache_len).to(dev)
    outs = []
    for _ in range(2):
        kbar = sa.build_block_summary(kc, cl, block_k=64)
        o, lse, sel = sa.sparse_decode(q, kc, vc, kbar, cl, block_k=64, top_k=24 if top_p == 0 else 64,
                                       sink=32, local=256, top_p=top_p)
        torch.cuda.synchronize()
        outs.append((kbar.cpu(), o.cpu(), lse.cpu(), sel.cpu()))
    for a_, b_ in zip(*outs):
        assert torch.equal(a_.view(torch.int16) if a_.dtype == torch.bfloat16 else a_,
                           b_.view(torch.int16) if b_.dtype == torch.bfloat16 else b_)


@pytest.mark.parametrize("granularity,bq,bk", [("block", 128, 64), ("block", 64, 64),
                                               ("stripe", 128, 64), ("block", 64, 32),
                                               ("block", 128, 32)])
def test_prefill_arbitrary_lists(dev, granularity, bq, bk):
    """Lists a caller builds itself (not from the estimate): random ascending subsets that
    include entries past the diagonal (ignored: only j <= r counts), empty lists, and lists
    whose entries all lie in a row's future.  Rows that see no key get O = 0 and LSE = -inf;
    every other row matches the oracle's attention over its visible listed tokens."""
    import torch
    import block_sparse_attention_estimate_amd as sa
    name = "stripe_64k" if granularity == "stripe" else "llama8b_32k"
    x = synth.make_prefill(name, seq=1500, hq=8, hkv=2)
    B, N, Hq, D = x.q.shape
    Hkv, G = 2, 4
    nqb, nkb = -(-N // bq), -(-N // bk)
    rng = np.random.default_rng(21)
    ref_lists = {}
    for g in range(Hkv):
        for i in range(nqb):
            kind = rng.integers(0, 4)
            ncand = nkb if granularity == "block" else N
            if kind == 0:
                kept = np.zeros(0, np.int64)                       # empty
            elif kind == 1:                                        # only the far future
                r1 = min(N, (i + 1) * bq)
                lo = r1 // bk + 1 if granularity == "block" else r1 + 5
                kept = np.arange(lo, ncand) if lo < ncand else np.zeros(0, np.int64)
            else:                                                  # random, incl. future
                kept = np.nonzero(rng.random(ncand) < rng.uniform(0.02, 0.6))[0]
            ref_lists[(0, g, i)] = kept.astype(np.int64)
    stride = nkb if granularity == "block" else N
    counts = np.zeros((1, Hkv, nqb), np.int32)
    idx = np.zeros((1, Hkv, nqb, stride), np.int32)
    for (b, g, i), kept in ref_lists.items():
        counts[b, g, i] = kept.size
        idx[b, g, i, :kept.size] = kept
    lists = sa.Lists(torch.from_numpy(counts).to(dev), torch.from_numpy(idx).to(dev), stride,
                     granularity)
    q, k, v = to_dev(x.q, dev), to_dev(x.k, dev), to_dev(x.v, dev)
    o, lse = sa.sparse_prefill(q, k, v, lists, block_q=bq, block_k=bk, sink=32, local=256)
    torch.cuda.synchronize()
    og = o.float().cpu().numpy()
    lg = lse.cpu().numpy()
    def toks_of(b, h, i):
        kept = ref_lists[(b, h // G, i)]
        t = kept if granularity == "stripe" else (kept[:, None] * bk + np.arange(bk)).ravel()
        return t[t < N]
    rows = [(0, h, i) for h in range(Hq) for i in range(nqb)]
    # the oracle's plain definition needs some listed token in range; blocks without one are
    # checked as rows without keys below
    with_toks = [(b, h, i) for (b, h, i) in rows if toks_of(b, h, i).size > 0]
    with np.errstate(invalid="ignore", divide="ignore"):
        res = oracle.attention_rows(x.q, x.k, x.v, ref_lists, block_q=bq, block_k=bk,
                                    granularity=granularity, rows=with_toks)
    n_empty = 0
    errs = []
    for (b, h, i) in rows:
        r0, r1 = i * bq, min(N, (i + 1) * bq)
        toks = toks_of(b, h, i)
        oref, lref = res.get((b, h, i), (None, None))
        for t, r in enumerate(range(r0, r1)):
            if not np.any(toks <= r):
                n_empty += 1
                assert np.all(og[b, r, h] == 0.0) and lg[b, h, r] == -np.inf, (b, h, r)
            else:
                errs.append(np.abs(og[b, r, h] - oref[t]))
                assert abs(lg[b, h, r] - lref[t]) < 1e-2, (b, h, r)
    err = np.concatenate(errs)
    log(f"  arbitrary {granularity} bq={bq} bk={bk}: rows without keys {n_empty}, "
        f"max|dO|={err.max():.2e} mean={err.mean():.2e}")
    assert n_empty > 0 and err.max() < MAX_ABS and err.mean() < MEAN_ABS


@pytest.mark.parametrize("bk,top_k,top_p,summary", [(64, 8, 0.0, "bf16"), (64, 40, 0.0, "bf16"),
                                                     (32, 12, 0.0, "bf16"), (64, 40, 0.6, "bf16"),
                                                     (64, 8, 0.0, "q4"), (64, 8, 0.0, "fp4")])
def test_decode_edge_lengths(dev, bk, top_k, top_p, summary):
    """Cache lengths at the edges: one token, the sink boundary, block boundaries, the window
    boundary and a full cache, in one batch (selection, summaries and attention)."""
    import torch
    import block_sparse_attention_estimate_amd as sa
    lens = [1, 31, 32, 63, 64, 65, 257, 300, 2048]
    x = synth.make_decode(batch=len(lens), seq=2048, hq=8, hkv=2, head_dim=128, top_k=top_k)
    x.cache_len[:] = np.array(lens, np.int32)
    q, kc, vc = to_dev(x.q, dev), to_dev(x.k_cache, dev), to_dev(x.v_cache, dev)
    cl = torch.from_numpy(x.cache_len).to(dev)
    kbar = sa.build_block_summary(kc, cl, block_k=bk)
    summ = kbar
    if summary == "q4":
        summ = sa.quantize_block_summary(kbar, block_k=bk)
    elif summary == "fp4":
        summ = sa.quantize_block_summary_fp4(kbar, block_k=bk)
    o, lse, sel = sa.sparse_decode(q, kc, vc, summ, cl, block_k=bk, top_k=top_k, sink=32, local=256,
                                   top_p=top_p)
    torch.cuda.synchronize()
    kbar_ref = oracle.block_summary(x.k_cache, x.cache_len, bk)
    kb = kbar.view(torch.int16).cpu().numpy().view(np.uint16)
    for b, L in enumerate(lens):
        nb = -(-L // bk)
        np.testing.assert_array_equal(kb[b, :nb], kbar_ref[b, :nb])
    score_src = kbar_ref
    if summary == "q4":
        score_src = oracle.dequantize_summary_q4(*oracle.quantize_summary_q4(kbar_ref))
    elif summary == "fp4":
        score_src = oracle.dequantize_summary_fp4(*oracle.quantize_summary_fp4(kbar_ref))
    ref = oracle.decode_select(x.q, score_src, x.cache_len, block_k=bk, top_k=top_k, sink=32,
                               local=256, top_p=top_p)
    s = sel.cpu().numpy()
    if top_p > 0:
        used, off, flips = check_topp_selection(s, ref)
    else:
        used, flips = {}, 0
        for (b, g), r in ref.items():
            k_ = min(top_k, -(-lens[b] // bk))
            got = s[b, g, :k_]
            assert (s[b, g, k_:] == -1).all() and np.all(np.diff(got) > 0)
            diff = set(got.tolist()) ^ set(r["selected"].tolist())
            assert diff <= set(r["ambiguous"].tolist()), ((b, g), sorted(diff))
            flips += len(diff)
            used[(b, g)] = got
    O, LSE = oracle.decode_attention(x.q, x.k_cache, x.v_cache, x.cache_len, used, block_k=bk)
    err = np.abs(o.float().cpu().numpy() - O)
    assert err.max() < MAX_ABS and err.mean() < MEAN_ABS, (err.max(), err.mean())
    assert np.abs(lse.cpu().numpy() - LSE).max() < 1e-2
    log(f"  decode edge lengths bk={bk} K={top_k} top_p={top_p}: flips={flips} max|dO|={err.max():.2e}")


@pytest.mark.parametrize("top_p", [0.0, 0.5])
def test_decode_empty_cache(dev, top_p):
    """A cache of length 0 beside non-empty ones: nothing is selected for it, its output is 0
    and its LSE -inf (the documented result for an empty cache); the other sequences of the
    batch meet the usual bars against the oracle."""
    import torch
    import block_sparse_attention_estimate_amd as sa
    lens = [0, 40, 700]
    x = synth.make_decode(batch=len(lens), seq=1024, hq=8, hkv=2, head_dim=128, top_k=8)
    x.cache_len[:] = np.array(lens, np.int32)
    log(f"decode empty cache top_p={top_p}")
    q, kc, vc = to_dev(x.q, dev), to_dev(x.k_cache, dev), to_dev(x.v_cache, dev)
    cl = torch.from_numpy(x.cache_len).to(dev)
    kbar = sa.build_block_summary(kc, cl, block_k=64)
    o, lse, sel = sa.sparse_decode(q, kc, vc, kbar, cl, block_k=64, top_k=8, sink=32, local=256,
                                   top_p=top_p)
    torch.cuda.synchronize()
    assert (kbar[0] == 0).all()
    assert (o[0].float() == 0).all()
    assert torch.isneginf(lse[0]).all()
    assert (sel[0] == -1).all()
    kbar_ref = oracle.block_summary(x.k_cache[1:], x.cache_len[1:], 64)
    ref = oracle.decode_select(x.q[1:], kbar_ref, x.cache_len[1:], block_k=64, top_k=8, sink=32,
                               local=256, top_p=top_p)
    s = sel.cpu().numpy()[1:]
    if top_p > 0:
        used, _, _ = check_topp_selection(s, ref)
    else:
        used = {}
        for (b, g), r in ref.items():
            k_ = min(8, -(-lens[b + 1] // 64))
            got = s[b, g, :k_]
            diff = set(got.tolist()) ^ set(r["selected"].tolist())
            assert diff <= set(r["ambiguous"].tolist()), ((b, g), sorted(diff))
            used[(b, g)] = got
    O, LSE = oracle.decode_attention(x.q[1:], x.k_cache[1:], x.v_cache[1:], x.cache_len[1:], used,
                                     block_k=64)
    err = np.abs(o[1:].float().cpu().numpy() - O)
    assert err.max() < MAX_ABS and err.mean() < MEAN_ABS, (err.max(), err.mean())
    assert np.abs(lse[1:].cpu().numpy() - LSE).max() < 1e-2
