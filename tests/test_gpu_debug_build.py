"""Diagnostics.  The debug build (libsa_debug.so): on valid inputs it returns the release
build's results bit for bit; on caller data that the release kernels clamp -- a list count past
the stride, a list entry outside the sequence, entries out of order, a cache length past the
cache -- the release build still runs (memory-safe, status ok) and the debug build reports
SA_ERR_CHECK with the matching sa_debug_flags() bits.  SA_LOG: each entry point prints its
configuration line to stderr."""
import numpy as np
import pytest

import synth
from helpers import log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    import block_sparse_attention_estimate_amd as sa
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sa.load_library()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def dbg_lib(dev):
    from block_sparse_attention_estimate_amd import _lib
    return _lib.open_library(_lib.DEBUG_LIB_PATH)


def _with_lib(monkeypatch, lib, fn):
    """Run fn with the binding's entry points bound to lib (the debug build)."""
    from block_sparse_attention_estimate_amd import _lib
    with monkeypatch.context() as m:
        m.setattr(_lib, "_lib", lib)
        return fn()


def _status(fn):
    """The status of fn's call: 0 when it returns, else the SaError's status."""
    import block_sparse_attention_estimate_amd as sa
    try:
        fn()
        return 0
    except sa.SaError as e:
        return e.status


def _copy_lists(lists):
    import block_sparse_attention_estimate_amd as sa
    return sa.Lists(counts=lists.counts.clone(), idx=lists.idx.clone(), stride=lists.stride,
                    granularity=lists.granularity)


@pytest.mark.parametrize("gran", ["block", "stripe"])
def test_debug_prefill(dev, dbg_lib, monkeypatch, gran):
    import torch
    import block_sparse_attention_estimate_amd as sa
    from block_sparse_attention_estimate_amd import _lib
    name = "stripe_64k" if gran == "stripe" else "llama8b_32k"
    x = synth.make_prefill(name, seq=1500, hq=8, hkv=2)
    log(f"debug build prefill {gran} N={x.q.shape[1]}")
    q, k, v = to_dev(x.q, dev), to_dev(x.k, dev), to_dev(x.v, dev)
    kw = dict(block_q=x.block_q, block_k=x.block_k, sink=x.sink, local=x.local)
    lists = sa.estimate_mask(q, k, np.full(8, 6.0, np.float32), granularity=gran, **kw)
    o_rel, lse_rel = sa.sparse_prefill(q, k, v, lists, **kw)
    o_dbg, lse_dbg = _with_lib(monkeypatch, dbg_lib, lambda: sa.sparse_prefill(q, k, v, lists, **kw))
    torch.cuda.synchronize()
    assert torch.equal(o_dbg, o_rel) and torch.equal(lse_dbg, lse_rel)

    counts = lists.counts.cpu().numpy()
    B, Hkv, nqb = counts.shape
    i = nqb - 1                                      # the last query block has the most entries
    assert counts[0, 0, i] >= 2
    lim = x.q.shape[1] if gran == "stripe" else -(-x.q.shape[1] // x.block_k)
    cases = []
    bad = _copy_lists(lists)
    bad.idx[0, 0, i, counts[0, 0, i] - 1] = lim       # one past the sequence's last block / column
    cases.append(("entry out of range", bad, _lib.SA_DBG_RANGE))
    bad = _copy_lists(lists)
    first, second = int(lists.idx[0, 1, i, 0]), int(lists.idx[0, 1, i, 1])
    bad.idx[0, 1, i, 0], bad.idx[0, 1, i, 1] = second, first
    cases.append(("entries out of order", bad, _lib.SA_DBG_ORDER))
    bad = _copy_lists(lists)
    bad.counts[0, 0, 0] = lists.stride + 1
    cases.append(("count past the stride", bad, _lib.SA_DBG_COUNT))
    bad = _copy_lists(lists)
    bad.idx[0, 1, i, 0] = -1
    cases.append(("negative entry", bad, _lib.SA_DBG_RANGE))
    for what, bad, bit in cases:
        log(f"  {what}")
        o, _ = sa.sparse_prefill(q, k, v, bad, **kw)     # release: clamps, runs, status ok
        torch.cuda.synchronize()
        assert torch.isfinite(o.float()).all(), what
        st = _status(lambda: _with_lib(monkeypatch, dbg_lib, lambda: sa.sparse_prefill(q, k, v, bad, **kw)))
        assert st == _lib.SA_ERR_CHECK, (what, st)
        assert dbg_lib.sa_debug_flags() & bit, (what, dbg_lib.sa_debug_flags())
    # the check word is cleared after a failing call: valid lists pass again
    st = _status(lambda: _with_lib(monkeypatch, dbg_lib, lambda: sa.sparse_prefill(q, k, v, lists, **kw)))
    assert st == 0


def test_debug_decode(dev, dbg_lib, monkeypatch):
    import torch
    import block_sparse_attention_estimate_amd as sa
    from block_sparse_attention_estimate_amd import _lib
    d = synth.make_decode(batch=2, seq=3000, hq=8, hkv=2, head_dim=128, top_k=16)
    log("debug build decode")
    qd, kc, vc = (to_dev(a, dev) for a in (d.q, d.k_cache, d.v_cache))
    cl = torch.from_numpy(d.cache_len).to(dev)
    kw = dict(block_k=64, top_k=16, sink=32, local=256)
    kbar = sa.build_block_summary(kc, cl, block_k=64)
    ref = sa.sparse_decode(qd, kc, vc, kbar, cl, **kw)

    def run():
        kb = sa.build_block_summary(kc, cl, block_k=64)
        return kb, sa.sparse_decode(qd, kc, vc, kb, cl, **kw)
    kb_dbg, got = _with_lib(monkeypatch, dbg_lib, run)
    torch.cuda.synchronize()
    assert torch.equal(kb_dbg, kbar)
    for a, b in zip(got, ref):
        assert torch.equal(a, b)

    L = kc.shape[1]
    for bad_len in (L + 5,):                          # clamped to L by the release kernels
        log(f"  cache length {bad_len}")
        bad = cl.clone()
        bad[0] = bad_len
        o, _, _ = sa.sparse_decode(qd, kc, vc, kbar, bad, **kw)   # release: clamped, status ok
        torch.cuda.synchronize()
        assert torch.isfinite(o.float()).all()
        for call in (lambda: sa.build_block_summary(kc, bad, block_k=64),
                     lambda: sa.sparse_decode(qd, kc, vc, kbar, bad, **kw)):
            st = _status(lambda: _with_lib(monkeypatch, dbg_lib, call))
            assert st == _lib.SA_ERR_CHECK, (bad_len, st)
            assert dbg_lib.sa_debug_flags() & _lib.SA_DBG_CACHE_LEN


def test_sa_log_lines(dev, monkeypatch, capfd):
    import torch
    import block_sparse_attention_estimate_amd as sa
    x = synth.make_prefill("llama8b_32k", seq=600, hq=8, hkv=2)
    q, k, v = to_dev(x.q, dev), to_dev(x.k, dev), to_dev(x.v, dev)
    kw = dict(block_q=x.block_q, block_k=x.block_k, sink=x.sink, local=x.local)
    theta = np.full(8, 6.0, np.float32)
    capfd.readouterr()
    monkeypatch.setenv("SA_LOG", "1")
    lists = sa.estimate_mask(q, k, theta, **kw)
    sa.sparse_prefill(q, k, v, lists, **kw)
    d = synth.make_decode(batch=2, seq=1000, hq=8, hkv=2, head_dim=128, top_k=8)
    qd, kc, vc = (to_dev(a, dev) for a in (d.q, d.k_cache, d.v_cache))
    cl = torch.from_numpy(d.cache_len).to(dev)
    kbar = sa.build_block_summary(kc, cl, block_k=64)
    sa.sparse_decode(qd, kc, vc, kbar, cl, block_k=64, top_k=8, sink=32, local=256)
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    lines = [ln for ln in err.splitlines() if ln.startswith("[sa] ")]
    assert len(lines) == 4, err
    assert lines[0].startswith("[sa] sa_estimate_mask: B=1 Hq=8 Hkv=2 d=128 N=600 head_map=h/G "
                               f"block_q={x.block_q} block_k=64 sink={x.sink} local={x.local} "
                               "granularity=block estimator=pooled step=1"), lines[0]
    assert lines[1].startswith("[sa] sa_sparse_prefill: B=1 Hq=8 Hkv=2 d=128 N=600"), lines[1]
    assert f"row_tiles_per_block={x.block_q // 64}" in lines[1]
    assert lines[2].startswith("[sa] sa_build_block_summary: B=2 Hq=2 Hkv=2 d=128 L=1000 block_k=64")
    assert lines[3].startswith("[sa] sa_sparse_decode: B=2 Hq=8 Hkv=2 d=128 L=1000 block_k=64 top_k=8")
    assert "summary=bf16" in lines[3]
    monkeypatch.setenv("SA_LOG", "0")
    sa.sparse_prefill(q, k, v, lists, **kw)
    torch.cuda.synchronize()
    assert "[sa]" not in capfd.readouterr().err
