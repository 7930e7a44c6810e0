"""Pins of the oracle's per-head threshold calibration (CPU only).

The error is pinned against an independent route (torch's scaled_dot_product_attention in
float64 under an explicit boolean mask built from the lists, summed by torch); the loop is
pinned by its closed-form cases: no halvings allowed returns theta = -ln(tau0); an
unreachable-never bound never halves; a zero bound halves exactly until the estimate keeps
every causal block, where the error is exactly zero (theta = +inf keeps every block, which
the attention pins tie to dense causal attention).
"""
import math

import numpy as np
import torch

import oracle
import synth

KW = dict(block_q=64, block_k=64, sink=32, local=128)


def _inputs(seed=3, N=768, Hq=4, Hkv=2, D=32):
    x = synth.make_prefill("llama8b_32k", seed=seed, seq=N, hq=Hq, hkv=Hkv, head_dim=D)
    return x.q, x.k, x.v


def _mask_from_lists(lists, b, g, N, bq, bk):
    m = np.zeros((N, N), dtype=bool)
    for i in range(-(-N // bq)):
        r0, r1 = i * bq, min(N, (i + 1) * bq)
        for J in lists[(b, g, i)]:
            m[r0:r1, J * bk:min(N, (J + 1) * bk)] = True
    return m & np.tril(np.ones((N, N), dtype=bool))


def test_full_lists_match_theta_inf():
    q, k, v = _inputs()
    N = q.shape[1]
    est = oracle.estimate_all(q, k, np.full(q.shape[2], np.inf), granularity="block", **KW)
    full = oracle.full_lists(N, 1, k.shape[2], KW["block_q"], KW["block_k"])
    assert set(est) == set(full)
    for key in full:
        np.testing.assert_array_equal(est[key]["kept"], full[key])


def test_error_against_sdpa():
    q, k, v = _inputs()
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    theta = np.full(Hq, 11.0, dtype=np.float32)
    est = oracle.estimate_all(q, k, theta, granularity="block", keep_margins=False, **KW)
    lists = {key: r["kept"] for key, r in est.items()}
    kw = dict(block_q=KW["block_q"], block_k=KW["block_k"])
    o_ref, _ = oracle.attention_all(q, k, v, oracle.full_lists(N, B, Hkv, **kw), **kw)
    o_sp, _ = oracle.attention_all(q, k, v, lists, **kw)
    err = oracle.head_l1_error(o_ref, o_sp)
    # independent: SDPA dense causal and SDPA under the list mask, L1 summed by torch
    qf, kf, vf = (torch.from_numpy(synth.bf16_bits_to_f64(t)[0]) for t in (q, k, v))
    c = float(oracle.softmax_scale(D))
    for h in range(Hq):
        g = h // (Hq // Hkv)
        qt, kt, vt = qf[:, h, :][None], kf[:, g, :][None], vf[:, g, :][None]
        dense = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=c)
        m = torch.from_numpy(_mask_from_lists(lists, 0, g, N, KW["block_q"], KW["block_k"]))
        sparse = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=c)
        ref = float((dense - sparse).abs().sum()) / N
        assert abs(err[h] - ref) <= 1e-10 * max(1.0, ref), (h, err[h], ref)
    assert (err > 0).any(), "the test needs a mask that drops something"


def test_no_halvings_returns_theta0():
    q, k, v = _inputs()
    r = oracle.calibrate_theta(q, k, v, tau0=0.008, err_bound=1e-9, max_halvings=0, **KW)
    assert np.all(r["theta"] == np.float32(-math.log(0.008)))
    assert np.all(r["halvings"] == 0) and len(r["history"]) == 1


def test_loose_bound_never_halves():
    q, k, v = _inputs()
    r = oracle.calibrate_theta(q, k, v, tau0=0.008, err_bound=1e9, max_halvings=5, **KW)
    assert np.all(r["halvings"] == 0)


def test_zero_bound_stops_at_full_lists():
    q, k, v = _inputs()
    r = oracle.calibrate_theta(q, k, v, tau0=1e-16, err_bound=1e-300, max_halvings=40, **KW)
    # every head reached error exactly zero (its group keeps every causal block) ...
    assert np.all(r["err"] == 0.0)
    assert np.all(r["halvings"] < 40)
    # ... and the round before its last halving it was not yet zero
    for h, kh in enumerate(r["halvings"]):
        if kh > 0:
            hist = [e[h] for th, e in r["history"]]
            assert hist[-1] == 0.0
            assert any(x > 0 for x in hist[:-1])
    # the thetas are -ln(tau0) + k ln 2, rounded once to fp32
    want = np.array([-math.log(1e-16) + kh * math.log(2.0) for kh in r["halvings"]], dtype=np.float32)
    np.testing.assert_array_equal(r["theta"], want)


def test_head_map_permutes_the_calibration():
    """Reordering the query heads of Q, with the head map reordered alike, reorders the
    calibrated thetas, halvings and errors alike (the map reaches the estimate and the
    attention of every round); a map that ignored the reordering would pair heads with the
    wrong KV head and change them."""
    q, k, v = _inputs(seed=5, N=1536, Hq=8, Hkv=2, D=32)
    # a short window and a large tau0 so the estimate drops blocks and the heads' errors differ
    kw = dict(block_q=64, block_k=64, sink=16, local=64, tau0=0.5, err_bound=2e-4,
              max_halvings=3)
    base = oracle.calibrate_theta(q, k, v, **kw)
    perm = np.array([5, 0, 7, 2, 1, 6, 3, 4])
    kv_of_q = perm // 4                            # the KV head of the reordered head j
    got = oracle.calibrate_theta(q[:, :, perm, :], k, v, kv_of_q=kv_of_q, **kw)
    np.testing.assert_array_equal(got["halvings"], base["halvings"][perm])
    np.testing.assert_array_equal(got["theta"], base["theta"][perm])
    np.testing.assert_allclose(got["err"], base["err"][perm], rtol=0, atol=1e-12)
    assert len(set(base["halvings"].tolist())) > 1    # the heads differ, so the order shows
    wrong = oracle.calibrate_theta(q[:, :, perm, :], k, v, **kw)   # default map, wrong pairing
    assert not np.allclose(wrong["err"], base["err"][perm], atol=1e-6)
