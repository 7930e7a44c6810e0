"""Pins of the oracle's masked attention and decode (CPU only).

theta = +inf (every causal block kept) must reproduce dense causal attention computed by an
independent library routine (torch's scaled_dot_product_attention on CPU in float64);
theta = -inf must reproduce the same routine under an explicit boolean mask built from the
token-level sink + local-window definition (the sliding-window special case).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_arithmetic.json")


def _sdpa(q, k, v, c, mask=None, causal=False):
    """q [N, Hq, d], k/v [N, Hkv, d] float64 -> O [N, Hq, d], via torch (GQA by repeat)."""
    N, Hq, D = q.shape
    Hkv = k.shape[1]
    rep = Hq // Hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(np.repeat(k, rep, axis=1)).permute(1, 0, 2)
    vt = torch.from_numpy(np.repeat(v, rep, axis=1)).permute(1, 0, 2)
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m,
                                                         is_causal=causal, scale=float(c))
    return o.permute(1, 0, 2).numpy()


def _inputs(seed, N, Hq, Hkv, D):
    rng = np.random.default_rng(seed)
    mk = lambda s: synth.bf16_round_bits(rng.standard_normal(s).astype(np.float32))
    return mk((1, N, Hq, D)), mk((1, N, Hkv, D)), mk((1, N, Hkv, D))


@pytest.mark.parametrize("gran", ["block", "stripe"])
@pytest.mark.parametrize("N,bq,bk", [(256, 64, 32), (200, 32, 64), (130, 64, 64)])
def test_theta_inf_is_dense_causal(gran, N, bq, bk):
    q, k, v = _inputs(N, N, 4, 2, 32)
    kw = dict(block_q=bq, block_k=bk, sink=16, local=48, granularity=gran)
    est = oracle.estimate_all(q, k, np.full(4, np.inf), **kw)
    lists = {key: r["kept"] for key, r in est.items()}
    O, LSE = oracle.attention_all(q, k, v, lists, block_q=bq, block_k=bk, granularity=gran)
    qf, kf, vf = (synth.bf16_bits_to_f64(x)[0] for x in (q, k, v))
    c = oracle.softmax_scale(32)
    ref = _sdpa(qf, kf, vf, c, causal=True)
    np.testing.assert_allclose(O[0], ref, rtol=0, atol=1e-12)
    # LSE: exp(z - LSE) sums to one over the causal keys of every row.
    for h in range(4):
        z = float(c) * (qf[:, h, :] @ kf[:, h // 2, :].T)
        z = np.where(np.tril(np.ones((N, N), bool)), z, -np.inf)
        np.testing.assert_allclose(np.exp(z - LSE[0, h][:, None]).sum(axis=1), 1.0, atol=1e-12)


@pytest.mark.parametrize("N,bq,bk,sink,local", [(320, 64, 32, 16, 48), (257, 32, 64, 8, 100)])
def test_theta_minus_inf_is_banded(N, bq, bk, sink, local):
    q, k, v = _inputs(7 + N, N, 2, 1, 16)
    est = oracle.estimate_all(q, k, np.full(2, -np.inf), block_q=bq, block_k=bk, sink=sink,
                              local=local)
    lists = {key: r["kept"] for key, r in est.items()}
    O, _ = oracle.attention_all(q, k, v, lists, block_q=bq, block_k=bk)
    # Token mask: key j is visible to row r when j <= r and j's block holds a token that is a
    # sink token or lies in the local window of some row of r's query block.
    mask = np.zeros((N, N), dtype=bool)
    for r in range(N):
        r0 = (r // bq) * bq
        e = min(N, r0 + bq) - 1
        for j in range(r + 1):
            J = j // bk
            toks = range(J * bk, min(N, (J + 1) * bk))
            if any(t <= e and (t < sink or t >= r0 - local + 1) for t in toks):
                mask[r, j] = True
    qf, kf, vf = (synth.bf16_bits_to_f64(x)[0] for x in (q, k, v))
    ref = _sdpa(qf, kf, vf, oracle.softmax_scale(16), mask=mask)
    np.testing.assert_allclose(O[0], ref, rtol=0, atol=1e-12)


def test_decode_full_selection_is_dense_last_row():
    x = synth.make_decode(batch=2, seq=1000, hq=4, hkv=2, head_dim=32, top_k=64)
    kbar = oracle.block_summary(x.k_cache, x.cache_len, 64)
    sel = oracle.decode_select(x.q, kbar, x.cache_len, block_k=64, top_k=64, sink=32, local=256)
    for key, r in sel.items():
        assert list(r["selected"]) == list(range(16))
    O, LSE = oracle.decode_attention(x.q, x.k_cache, x.v_cache, x.cache_len,
                                     {k_: r["selected"] for k_, r in sel.items()}, block_k=64)
    c = oracle.softmax_scale(32)
    for b in range(2):
        qf = synth.bf16_bits_to_f64(x.q[b])[None]                  # [1, Hq, d]
        kf = synth.bf16_bits_to_f64(x.k_cache[b])
        vf = synth.bf16_bits_to_f64(x.v_cache[b])
        # the query is the last row: it sees every cached token
        ref = _sdpa(qf, kf, vf, c)
        np.testing.assert_allclose(O[b], ref[0], rtol=0, atol=1e-12)


def test_decode_selection_rules():
    x = synth.make_decode(batch=3, seq=5000, hq=4, hkv=2, head_dim=32, top_k=24)
    x.cache_len[1] = 4097            # ragged cache lengths
    x.cache_len[2] = 900
    kbar = oracle.block_summary(x.k_cache, x.cache_len, 64)
    # summaries: nearest bf16 of the fp64 mean (torch's own float32 -> bfloat16 rounding)
    for b in range(3):
        lb = int(x.cache_len[b])
        for J in range(-(-lb // 64)):
            blk = synth.bf16_bits_to_f64(x.k_cache[b, J * 64:min(lb, J * 64 + 64)])
            mean32 = torch.from_numpy(blk.mean(axis=0).astype(np.float32))
            want = mean32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            np.testing.assert_array_equal(kbar[b, J], want)
    sel = oracle.decode_select(x.q, kbar, x.cache_len, block_k=64, top_k=24, sink=32, local=256)
    for (b, g), r in sel.items():
        nkb = -(-int(x.cache_len[b]) // 64)
        s = list(r["selected"])
        assert s == sorted(set(s)) and len(s) == min(24, nkb)
        assert set(r["forced"]) <= set(s)
        lb = int(x.cache_len[b])
        assert 0 in s and (lb - 1) // 64 in s and (lb - 256) // 64 in s
        if nkb > 24:
            picked = [J for J in s if J not in set(r["forced"])]
            others = [J for J in range(nkb) if J not in set(s)]
            worst = min(r["score"][J] for J in picked)
            assert all(r["score"][J] <= worst for J in others)


def test_page_arithmetic_pins():
    gold = json.load(open(GOLDEN))
    pm = gold["pruned_mass"]
    n, gap = pm["n_keys"], pm["gap_logits"]
    logits = np.concatenate([[0.0], np.full(n, -gap)])
    kept = np.zeros(n + 1, bool)
    kept[0] = True
    # every tail key fails a - s <= theta (gap 13 > theta 12) and is pruned
    assert gap > pm["theta"]
    frac = oracle.pruned_mass_fraction(logits, kept)
    assert abs(frac / (1 - frac) - pm["relative_mass"]) < 5e-4
    assert abs(frac - pm["mass_fraction"]) < 5e-3
    tb = gold["table1_block"]
    assert oracle.sparsity_from_kept(tb["top_k_blocks"] * tb["block_size"], tb["context_keys"]) == tb["sparsity"]
    ts = gold["table1_stripe"]
    assert oracle.sparsity_from_kept(ts["top_k_keys"], ts["context_keys"]) == ts["sparsity"]
    st = gold["sale_tau"]
    assert abs(-math.log(st["tau"]) - st["equivalent_logit_margin"]) < 5e-3
    rng = np.random.default_rng(0)
    s = rng.uniform(-10, 2, 1000)
    em, el = 1.5, rng.uniform(1, 5)
    direct = np.exp(s - em) / el >= st["tau"]
    np.testing.assert_array_equal(oracle.sale_log_margin(s, em, el, st["tau"]) >= 0, direct)
    # with a one-term sink-local area (el = 1) the SALE test is Eq. (2) with theta = -ln tau
    np.testing.assert_array_equal(oracle.sale_log_margin(s, em, 1.0, st["tau"]) >= 0,
                                  em - s <= -math.log(st["tau"]))
