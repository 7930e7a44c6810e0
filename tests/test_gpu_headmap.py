"""GPU parity with a GQA head map that is not h // G (sa_shape.kv_head_of_q): the query heads
of a KV head sit at scattered positions of Q and O.  The oracle takes the same map (kv_of_q);
lists, margins, attention, the anchor state, the resumed prefill and decode must meet the usual
bars, with per-query-head thetas so that a wrong permutation of theta would show."""
import numpy as np
import pytest

import oracle
import synth
from helpers import (MAX_ABS, MEAN_ABS, compare_lists, compare_outputs, lists_from_ref, log, to_dev,
                     upload_lists)

pytestmark = pytest.mark.gpu

# KV head of each query head: two groups of four, interleaved out of order
KV_OF_Q = np.array([1, 0, 0, 1, 1, 0, 1, 0], np.int32)


@pytest.fixture(scope="module")
def dev():
    import torch
    import block_sparse_attention_estimate_amd as sa
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sa.load_library()
    return torch.device("cuda:0")


def _margins_close(lists, ref):
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
    return worst


@pytest.mark.parametrize("estimator,gran", [("pooled", "block"), ("pooled", "stripe"),
                                            ("relative", "block"), ("relative_mxfp4", "block")])
def test_head_map_prefill(dev, estimator, gran):
    import torch
    import block_sparse_attention_estimate_amd as sa
    name = "stripe_64k" if gran == "stripe" else "llama8b_32k"
    x = synth.make_prefill(name, seq=1700, hq=8, hkv=2)
    B, N, Hq, D = x.q.shape
    # per-query-head thetas that keep more than the forced blocks at this size, and keep
    # different blocks under this map than under h // G
    theta = np.array([8.0, 14.0, 10.0, 12.0, 16.0, 9.0, 11.0, 20.0], np.float32)
    if estimator != "pooled":
        theta = theta - 4.0
    log(f"head map {KV_OF_Q.tolist()} {estimator} {gran} N={N}")
    q, k, v = to_dev(x.q, dev), to_dev(x.k, dev), to_dev(x.v, dev)
    kw = dict(block_q=x.block_q, block_k=x.block_k, sink=x.sink, local=x.local)
    lists = sa.estimate_mask(q, k, theta, granularity=gran, estimator=estimator, margins=True,
                             kv_head_of_q=KV_OF_Q, **kw)
    torch.cuda.synchronize()
    if estimator == "pooled":
        ref = oracle.estimate_all(x.q, x.k, theta, granularity=gran, kv_of_q=KV_OF_Q, **kw)
    else:
        lowbit = "mxfp4" if estimator == "relative_mxfp4" else "int8"
        ref = oracle.estimate_all_sale(x.q, x.k, theta, lowbit=lowbit, kv_of_q=KV_OF_Q, **kw)
    rows, entries, flips = compare_lists(lists, ref)
    worst = _margins_close(lists, ref)
    log(f"  lists ok: rows={rows} entries={entries} flips={flips} max|dmargin|={worst:.1e}")
    # the default map gives different lists here (the groups differ), so the map is in effect
    plain = sa.estimate_mask(q, k, theta, granularity=gran, estimator=estimator, **kw)
    torch.cuda.synchronize()
    assert not torch.equal(plain.counts, lists.counts)
    nqb = -(-N // x.block_q)
    dl = upload_lists(ref, (B, 2, nqb), dev, gran, lists.stride)
    o, lse = sa.sparse_prefill(q, k, v, dl, kv_head_of_q=KV_OF_Q, **kw)
    torch.cuda.synchronize()
    O, LSE = oracle.attention_all(x.q, x.k, x.v, lists_from_ref(ref), block_q=x.block_q,
                                  block_k=x.block_k, granularity=gran, kv_of_q=KV_OF_Q)
    mx, mean, lmax = compare_outputs(o, lse, O, LSE)
    log(f"  attention ok: max|dO|={mx:.2e} mean={mean:.2e} max|dLSE|={lmax:.2e}")


def test_head_map_anchor_state(dev):
    import torch
    import block_sparse_attention_estimate_amd as sa
    x = synth.make_prefill("llama8b_32k", seq=1300, hq=8, hkv=2)
    B, N, Hq, D = x.q.shape
    theta = np.array([8.0, 14.0, 10.0, 12.0, 16.0, 9.0, 11.0, 20.0], np.float32)
    q, k, v = to_dev(x.q, dev), to_dev(x.k, dev), to_dev(x.v, dev)
    kw = dict(block_q=128, block_k=64, sink=32, local=256)
    plain = sa.estimate_mask(q, k, theta, kv_head_of_q=KV_OF_Q, **kw)
    lists, st = sa.estimate_mask_anchor_state(q, k, v, theta, kv_head_of_q=KV_OF_Q, **kw)
    torch.cuda.synchronize()
    assert torch.equal(plain.counts, lists.counts)
    ref = oracle.estimate_all(x.q, x.k, theta, kv_of_q=KV_OF_Q, **kw)
    compare_lists(lists, ref)
    nqb = -(-N // 128)
    rows = [(0, h, i) for h in range(Hq) for i in range(nqb)]
    sref = oracle.anchor_state_rows(x.q, x.k, x.v, block_q=128, sink=32, local=256, rows=rows,
                                    kv_of_q=KV_OF_Q)
    so, sl = st.o.float().cpu().numpy(), st.lse.cpu().numpy()
    errs, lerrs = [], []
    for (b, h, i), (oa, la) in sref.items():
        r0, r1 = i * 128, min(N, (i + 1) * 128)
        errs.append(np.abs(so[b, r0:r1, h, :] - oa).ravel())
        lerrs.append(np.abs(sl[b, h, r0:r1] - la))
    err, lerr = np.concatenate(errs), np.concatenate(lerrs)
    assert err.max() < MAX_ABS and err.mean() < MEAN_ABS and lerr.max() < 1e-2
    dl = upload_lists(ref, (B, 2, nqb), dev, "block", lists.stride)
    o, lse = sa.sparse_prefill_resume(q, k, v, dl, st, kv_head_of_q=KV_OF_Q, **kw)
    torch.cuda.synchronize()
    O, LSE = oracle.attention_all(x.q, x.k, x.v, lists_from_ref(ref), block_q=128, block_k=64,
                                  kv_of_q=KV_OF_Q)
    mx, mean, lmax = compare_outputs(o, lse, O, LSE)
    log(f"  head-map anchor state ok: state max|dO|={err.max():.2e}; resumed max|dO|={mx:.2e}")


@pytest.mark.parametrize("summary", ["bf16", "q4", "fp4"])
def test_head_map_decode(dev, summary):
    import torch
    import block_sparse_attention_estimate_amd as sa
    x = synth.make_decode(batch=3, seq=4000, hq=8, hkv=2, head_dim=128, top_k=16)
    x.cache_len[1] = 4000 - 937
    q, kc, vc = to_dev(x.q, dev), to_dev(x.k_cache, dev), to_dev(x.v_cache, dev)
    cl = torch.from_numpy(x.cache_len).to(dev)
    kbar = sa.build_block_summary(kc, cl, block_k=64)
    kbar_ref = oracle.block_summary(x.k_cache, x.cache_len, 64)
    if summary == "q4":
        summ = sa.quantize_block_summary(kbar, block_k=64)
        c_ref, s_ref = oracle.quantize_summary_q4(kbar_ref)
        kref = oracle.dequantize_summary_q4(c_ref, s_ref)
    elif summary == "fp4":
        summ = sa.quantize_block_summary_fp4(kbar, block_k=64)
        vals, exps = oracle.quantize_summary_fp4(kbar_ref)
        kref = oracle.dequantize_summary_fp4(vals, exps)
    else:
        summ, kref = kbar, kbar_ref
    o, lse, sel = sa.sparse_decode(q, kc, vc, summ, cl, block_k=64, top_k=16, sink=32, local=256,
                                   kv_head_of_q=KV_OF_Q)
    torch.cuda.synchronize()
    ref = oracle.decode_select(x.q, kref, x.cache_len, block_k=64, top_k=16, sink=32, local=256,
                               kv_of_q=KV_OF_Q)
    s = sel.cpu().numpy()
    used, flips = {}, 0
    for (b, g), r in ref.items():
        k_ = min(16, -(-int(x.cache_len[b]) // 64))
        got = s[b, g, :k_]
        assert (s[b, g, k_:] == -1).all() and np.all(np.diff(got) > 0)
        diff = set(got.tolist()) ^ set(r["selected"].tolist())
        assert diff <= set(r["ambiguous"].tolist()), ((b, g), sorted(diff))
        flips += len(diff)
        used[(b, g)] = got
    O, LSE = oracle.decode_attention(x.q, x.k_cache, x.v_cache, x.cache_len, used, block_k=64,
                                     kv_of_q=KV_OF_Q)
    err = np.abs(o.float().cpu().numpy() - O)
    assert err.max() < MAX_ABS and err.mean() < MEAN_ABS, (err.max(), err.mean())
    assert np.abs(lse.cpu().numpy() - LSE).max() < 1e-2
    log(f"  head-map decode ({summary}) ok: flips={flips} max|dO|={err.max():.2e}")
