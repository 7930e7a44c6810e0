"""GPU parity with 32-key blocks (SALE's configuration: 64-row query blocks, 32-key blocks):
the three estimators' lists and margins against the oracle at block_k = 32 (one int8 key scale
per 32 keys), and the attention over the oracle's 32-key block lists (tiles pair listed blocks
from anywhere in the sequence; an odd list leaves the last tile half empty).  Caller-built
32-key lists with gaps, empty rows and future entries are in test_gpu_parity.py
(test_prefill_arbitrary_lists)."""
import numpy as np
import pytest

import oracle
import synth
from helpers import compare_lists, compare_outputs, lists_from_ref, log, to_dev, upload_lists

pytestmark = pytest.mark.gpu


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


@pytest.mark.parametrize("estimator", ["pooled", "relative", "relative_mxfp4"])
@pytest.mark.parametrize("seq,hq,hkv,d,bq", [(1500, 8, 2, 128, 64), (777, 4, 1, 64, 64),
                                             (2100, 4, 2, 128, 128)])
def test_block32_estimate_and_attention(dev, estimator, seq, hq, hkv, d, bq):
    import torch
    import block_sparse_attention_estimate_amd as sa
    x = synth.make_prefill("llama8b_32k", seq=seq, hq=hq, hkv=hkv, head_dim=d)
    B, N, Hq, D = x.q.shape
    grp = hq // hkv
    q, k, v = to_dev(x.q, dev), to_dev(x.k, dev), to_dev(x.v, dev)
    kw = dict(block_q=bq, block_k=32, sink=32, local=256)
    base = np.repeat(np.array([6.0, 10.0, 8.0, 14.0], np.float32)[:hkv], grp)
    if estimator != "pooled":
        base = base - 3.0
    lowbit = "mxfp4" if estimator == "relative_mxfp4" else "int8"
    for theta in [base, np.full(hq, -np.inf, np.float32), np.full(hq, np.inf, np.float32),
                  base + np.linspace(0, 2, hq, dtype=np.float32)]:
        log(f"bk32 {estimator} N={N} Hq={Hq} Hkv={hkv} d={D} bq={bq} theta={np.unique(theta)[:4]}")
        lists = sa.estimate_mask(q, k, theta, estimator=estimator, margins=True, **kw)
        torch.cuda.synchronize()
        if estimator == "pooled":
            ref = oracle.estimate_all(x.q, x.k, theta, **kw)
        else:
            ref = oracle.estimate_all_sale(x.q, x.k, theta, lowbit=lowbit, **kw)
        rows, entries, flips = compare_lists(lists, ref)
        worst = _margins_close(lists, ref)
        log(f"  lists ok: entries={entries} flips={flips} max|dmargin|={worst:.1e}")
    nqb = -(-N // bq)
    dl = upload_lists(ref, (B, hkv, nqb), dev, "block", lists.stride)
    o, lse = sa.sparse_prefill(q, k, v, dl, **kw)
    torch.cuda.synchronize()
    O, LSE = oracle.attention_all(x.q, x.k, x.v, lists_from_ref(ref), block_q=bq, block_k=32)
    mx, mean, lmax = compare_outputs(o, lse, O, LSE)
    log(f"  attention ok: max|dO|={mx:.2e} mean={mean:.2e} max|dLSE|={lmax:.2e}")


@pytest.mark.parametrize("seq", [1, 31, 32, 33, 65, 200, 1000])
def test_block32_edge_lengths(dev, seq):
    import torch
    import block_sparse_attention_estimate_amd as sa
    x = synth.make_prefill("llama8b_32k", seq=seq, hq=4, hkv=1)
    q, k, v = to_dev(x.q, dev), to_dev(x.k, dev), to_dev(x.v, dev)
    kw = dict(block_q=64, block_k=32, sink=32, local=256)
    theta = np.full(4, 8.0, np.float32)
    lists = sa.estimate_mask(q, k, theta, margins=True, **kw)
    torch.cuda.synchronize()
    ref = oracle.estimate_all(x.q, x.k, theta, **kw)
    compare_lists(lists, ref)
    _margins_close(lists, ref)
    nqb = -(-seq // 64)
    dl = upload_lists(ref, (1, 1, nqb), dev, "block", lists.stride)
    o, lse = sa.sparse_prefill(q, k, v, dl, **kw)
    torch.cuda.synchronize()
    O, LSE = oracle.attention_all(x.q, x.k, x.v, lists_from_ref(ref), block_q=64, block_k=32)
    compare_outputs(o, lse, O, LSE)
