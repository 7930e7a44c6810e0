"""Pins of the oracle's anchor-state reuse (CPU only).

* the anchor region against its closed-form size and against the forced blocks, which must
  contain it for every row of the query block (this is what makes resuming exact);
* the state in the special case sink = 0, local >= N (A(r) is every causal key) against
  torch's scaled_dot_product_attention on CPU in float64, and its LSE against torch's
  logsumexp;
* the state's LSE against the anchor of the estimate oracle (the max over the same tokens):
  x_a <= LSE_A <= x_a + ln |A(r)|;
* the merge of two disjoint partial attentions against attention over their union computed
  by torch, and resume = attention over the list (the plain definition in oracle.attention)
  on random lists that hold the forced blocks.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _inputs(seed, N, Hq, Hkv, D):
    rng = np.random.default_rng(seed)
    mk = lambda s: synth.bf16_round_bits(rng.standard_normal(s).astype(np.float32))
    return mk((1, N, Hq, D)), mk((1, N, Hkv, D)), mk((1, N, Hkv, D))


def _qrows(i, n, bq):
    return i * bq, min(n, (i + 1) * bq)


def _f(x):
    return synth.bf16_bits_to_f32(x).astype(np.float64)


@pytest.mark.parametrize("sink,local", [(0, 1), (32, 256), (64, 16), (5, 7), (300, 40)])
def test_region_size_and_coverage(sink, local):
    N, bq, bk = 700, 128, 64
    for r in range(N):
        A = oracle.anchor_region(r, sink, local)
        # closed form: the sink part plus the part of the window above the sink
        n_sink = min(sink, r + 1)
        lo = max(0, r - local + 1)
        n_win = max(0, r + 1 - max(lo, sink))
        assert A.size == n_sink + n_win
        assert A[-1] == r and np.all(np.diff(A) > 0)
    for i in range(-(-N // bq)):
        toks = set()
        for J in oracle.forced_blocks(i, N, bq, bk, sink, local):
            toks.update(range(J * bk, min(N, (J + 1) * bk)))
        r0, r1 = _qrows(i, N, bq)
        for r in range(r0, r1):
            assert set(oracle.anchor_region(r, sink, local).tolist()) <= toks


def test_state_dense_special_case():
    """sink = 0, local >= N: the anchor region is every causal key."""
    N, Hq, Hkv, D, bq = 200, 4, 2, 32, 64
    q, k, v = _inputs(3, N, Hq, Hkv, D)
    rows = [(0, h, i) for h in range(Hq) for i in range(-(-N // bq))]
    st = oracle.anchor_state_rows(q, k, v, block_q=bq, sink=0, local=N, rows=rows)
    c = float(oracle.softmax_scale(D))
    qt = torch.from_numpy(_f(q)[0]).permute(1, 0, 2)                       # [Hq, N, D]
    kt = torch.from_numpy(np.repeat(_f(k)[0], Hq // Hkv, axis=1)).permute(1, 0, 2)
    vt = torch.from_numpy(np.repeat(_f(v)[0], Hq // Hkv, axis=1)).permute(1, 0, 2)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=c)
    z = (qt @ kt.transpose(1, 2)) * c
    z = z.masked_fill(~torch.ones(N, N, dtype=torch.bool).tril(), float("-inf"))
    lse = torch.logsumexp(z, dim=-1)
    for (b, h, i), (oa, la) in st.items():
        r0, r1 = _qrows(i, N, bq)
        np.testing.assert_allclose(oa, o[h, r0:r1].numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(la, lse[h, r0:r1].numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("sink,local", [(32, 256), (8, 40), (0, 1)])
def test_state_lse_bounds_against_anchor(sink, local):
    N, Hq, Hkv, D, bq = 400, 2, 1, 64, 128
    q, k, v = _inputs(5, N, Hq, Hkv, D)
    c = float(oracle.softmax_scale(D))
    kf = _f(k)[0, :, 0, :]
    vf = _f(v)[0, :, 0, :]
    for h in range(Hq):
        for i in range(-(-N // bq)):
            r0, r1 = _qrows(i, N, bq)
            (oa, la), = oracle.anchor_state_rows(q, k, v, block_q=bq, sink=sink, local=local,
                                                 rows=[(0, h, i)]).values()
            xa = oracle.anchor_rows(_f(q)[0, r0:r1, h, :], kf, c, sink, local, r0, r1)
            sizes = np.array([oracle.anchor_region(r, sink, local).size for r in range(r0, r1)])
            assert np.all(la >= xa - 1e-12)
            assert np.all(la <= xa + np.log(sizes) + 1e-12)
            # O_A is a convex combination of the region's values
            for t, r in enumerate(range(r0, r1)):
                vv = vf[oracle.anchor_region(r, sink, local)]
                assert np.all(oa[t] >= vv.min(axis=0) - 1e-12)
                assert np.all(oa[t] <= vv.max(axis=0) + 1e-12)
            if local == 1 and sink == 0:        # A(r) = {r}: O_A = v_r, LSE_A = c q_r.k_r
                np.testing.assert_array_equal(oa, vf[r0:r1])
                np.testing.assert_allclose(la, xa, rtol=0, atol=0)


def test_merge_against_union():
    rng = np.random.default_rng(11)
    n, d = 57, 16
    z = rng.standard_normal((6, n)) * 3.0
    vv = rng.standard_normal((n, d))
    for trial in range(20):
        part = rng.random(n) < rng.uniform(0.05, 0.95)
        za = np.where(part[None, :], z, -np.inf)
        zb = np.where(~part[None, :], z, -np.inf)
        def attn(zz):
            t = torch.from_numpy(zz)
            p = torch.softmax(t, dim=-1).nan_to_num(0.0)
            return (p @ torch.from_numpy(vv)).numpy(), torch.logsumexp(t, dim=-1).numpy()
        oa, la = attn(za)
        ob, lb = attn(zb)
        o, lse = oracle.merge_partials(oa, la, ob, lb)
        ot, lt = attn(z)
        np.testing.assert_allclose(o, ot, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lt, rtol=0, atol=1e-12)
    # an empty second part returns the first unchanged
    o, lse = oracle.merge_partials(oa, la, np.zeros_like(oa), np.full(la.shape, -np.inf))
    np.testing.assert_array_equal(o, oa)
    np.testing.assert_array_equal(lse, la)


@pytest.mark.parametrize("sink,local,bq", [(32, 256, 128), (16, 100, 64), (70, 64, 128)])
def test_resume_equals_attention_over_list(sink, local, bq):
    N, Hq, Hkv, D, bk = 777, 4, 2, 32, 64
    q, k, v = _inputs(7, N, Hq, Hkv, D)
    rng = np.random.default_rng(8)
    nqb, nkb = -(-N // bq), -(-N // bk)
    lists = {}
    for g in range(Hkv):
        for i in range(nqb):
            r1 = min(N, (i + 1) * bq)
            cand = np.arange(-(-r1 // bk))
            pick = cand[rng.random(cand.size) < 0.4]
            lists[(0, g, i)] = np.union1d(pick, oracle.forced_blocks(i, N, bq, bk, sink, local))
    rows = [(0, h, i) for h in range(Hq) for i in range(nqb)]
    st = oracle.anchor_state_rows(q, k, v, block_q=bq, sink=sink, local=local, rows=rows)
    res = oracle.resume_rows(q, k, v, lists, st, block_q=bq, block_k=bk, sink=sink, local=local,
                             rows=rows)
    ref = oracle.attention_rows(q, k, v, lists, block_q=bq, block_k=bk, rows=rows)
    for key in rows:
        np.testing.assert_allclose(res[key][0], ref[key][0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(res[key][1], ref[key][1], rtol=0, atol=1e-12)
    assert nkb > 8


@pytest.mark.parametrize("sink,local,bq", [(32, 256, 128), (0, 100, 64), (70, 40, 128)])
def test_resume_equals_attention_over_column_list(sink, local, bq):
    """Column lists: the state over A(r) merged with the listed columns outside A(r) is the
    attention over the list when the list holds the forced columns (a superset of A(r)); the
    lists also hold columns past the block's last row, which no row may see."""
    N, Hq, Hkv, D = 700, 4, 2, 32
    q, k, v = _inputs(17, N, Hq, Hkv, D)
    rng = np.random.default_rng(18)
    nqb = -(-N // bq)
    lists = {}
    for g in range(Hkv):
        for i in range(nqb):
            cols = np.nonzero(rng.random(N) < 0.1)[0]              # any column, future ones too
            lists[(0, g, i)] = np.union1d(cols, oracle.forced_columns(i, N, bq, sink, local))
    rows = [(0, h, i) for h in range(Hq) for i in range(nqb)]
    st = oracle.anchor_state_rows(q, k, v, block_q=bq, sink=sink, local=local, rows=rows)
    res = oracle.resume_rows(q, k, v, lists, st, block_q=bq, block_k=64, sink=sink, local=local,
                             rows=rows, granularity="stripe")
    ref = oracle.attention_rows(q, k, v, lists, block_q=bq, block_k=64, rows=rows,
                                granularity="stripe")
    for key in rows:
        np.testing.assert_allclose(res[key][0], ref[key][0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(res[key][1], ref[key][1], rtol=0, atol=1e-12)
    # a planted mistake shows: resuming with the block reading of the same ids differs
    bad = oracle.resume_rows(q, k, v, lists, st, block_q=bq, block_k=64, sink=sink, local=local,
                             rows=rows[-1:])
    assert not np.allclose(bad[rows[-1]][0], ref[rows[-1]][0], atol=1e-6)


def test_resume_with_an_empty_list_returns_state():
    """An empty list (block or column) adds no token: the resume is the state itself."""
    N, Hq, Hkv, D, bq = 300, 2, 1, 32, 128
    q, k, v = _inputs(19, N, Hq, Hkv, D)
    nqb = -(-N // bq)
    rows = [(0, h, i) for h in range(Hq) for i in range(nqb)]
    st = oracle.anchor_state_rows(q, k, v, block_q=bq, sink=32, local=64, rows=rows)
    empty = {(0, 0, i): np.zeros(0, np.int64) for i in range(nqb)}
    for gran in ("block", "stripe"):
        res = oracle.resume_rows(q, k, v, empty, st, block_q=bq, block_k=64, sink=32, local=64,
                                 rows=rows, granularity=gran)
        for key in rows:
            np.testing.assert_allclose(res[key][0], st[key][0], rtol=0, atol=1e-15)
            np.testing.assert_array_equal(res[key][1], st[key][1])


def test_resume_without_rest_returns_state():
    """local >= N and sink = 0: every causal listed token is in A(r), the state is final."""
    N, Hq, Hkv, D, bq, bk = 300, 2, 1, 32, 128, 64
    q, k, v = _inputs(9, N, Hq, Hkv, D)
    nqb = -(-N // bq)
    lists = {(0, 0, i): oracle.forced_blocks(i, N, bq, bk, 0, N) for i in range(nqb)}
    rows = [(0, h, i) for h in range(Hq) for i in range(nqb)]
    st = oracle.anchor_state_rows(q, k, v, block_q=bq, sink=0, local=N, rows=rows)
    res = oracle.resume_rows(q, k, v, lists, st, block_q=bq, block_k=bk, sink=0, local=N, rows=rows)
    for key in rows:
        np.testing.assert_array_equal(res[key][0], st[key][0])
        np.testing.assert_array_equal(res[key][1], st[key][1])
    assert math.isfinite(float(st[rows[0]][1][0]))
