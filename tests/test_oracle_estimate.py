"""Pins of the oracle's estimation pass (CPU only).

The brute force below is written with plain Python loops and Python floats/ints, one
element at a time, straight from AnchorAttention Eq. (1)/(2) (anchor over the sink and
causal local window, block-averaged anchor and query, threshold compare with <=) and the
int8 symmetric quantiser; it shares nothing with the vectorised oracle.  Invariants cover
what brute force at tiny sizes cannot: key-shift and scale invariance, theta-nesting,
forced subset, stripe-within-block and union-over-heads.
"""
import math
import struct

import numpy as np
import pytest

import oracle
import synth


def f32(x: float) -> float:
    """Round a Python float to the nearest fp32 value (ties to even)."""
    return struct.unpack("f", struct.pack("f", x))[0]


def bf16_values(shape, rng, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return synth.bf16_round_bits(x)


def brute_force_lists(q, k, theta, *, bq, bk, sink, local, granularity="block"):
    """Pure-Python reference for the kept lists of every (b, g, i)."""
    qf = synth.bf16_bits_to_f64(q).tolist()
    kf = synth.bf16_bits_to_f64(k).tolist()
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    grp = Hq // Hkv
    c = f32(1.0 / math.sqrt(D))
    nqb = -(-N // bq)
    nkb = -(-N // bk)
    # int8 key tiles
    kq = {}
    sk = {}
    for b in range(B):
        for g in range(Hkv):
            for J in range(nkb):
                toks = range(J * bk, min(N, (J + 1) * bk))
                a = max(abs(f32(kf[b][t][g][d])) for t in toks for d in range(D))
                if a == 0.0:
                    sk[b, g, J] = 1.0
                    for t in toks:
                        kq[b, g, t] = [0] * D
                    continue
                inv = f32(127.0 / a)
                sk[b, g, J] = f32(a / 127.0)
                for t in toks:
                    kq[b, g, t] = [max(-127, min(127, round(f32(kf[b][t][g][d] * inv))))
                                   for d in range(D)]
    lists = {}
    for b in range(B):
        for g in range(Hkv):
            for i in range(nqb):
                r0, r1 = i * bq, min(N, (i + 1) * bq)
                e = r1 - 1
                if granularity == "block":
                    cands = [J for J in range(nkb) if J * bk <= e]
                else:
                    cands = list(range(e + 1))
                best = {x: -math.inf for x in cands}
                for h in range(g * grp, (g + 1) * grp):
                    # anchor per row, then its mean over the block
                    xs = []
                    for r in range(r0, r1):
                        m = -math.inf
                        for j in range(0, r + 1):
                            if j < sink or j >= r - local + 1:
                                s = c * sum(qf[b][r][h][d] * kf[b][j][g][d] for d in range(D))
                                m = max(m, s)
                        xs.append(m)
                    abar = sum(xs) / len(xs)
                    # pooled query, fp64 sum then fp32, fp32 division
                    qbar = [f32(f32(sum(qf[b][r][h][d] for r in range(r0, r1))) / f32(r1 - r0))
                            for d in range(D)]
                    a = max(abs(x) for x in qbar)
                    if a == 0.0:
                        sq, qq = 1.0, [0] * D
                    else:
                        inv = f32(127.0 / a)
                        sq = f32(a / 127.0)
                        qq = [max(-127, min(127, round(f32(x * inv)))) for x in qbar]
                    for x in cands:
                        cols = range(x * bk, min((x + 1) * bk, e + 1)) if granularity == "block" else [x]
                        E = -math.inf
                        for j in cols:
                            dot = sum(qq[d] * kq[b, g, j][d] for d in range(D))   # Python int
                            mult = f32(f32(sq * sk[b, g, j // bk]) * c)
                            E = max(E, f32(float(dot) * mult))
                        best[x] = max(best[x], E - (abar - float(theta[h])))
                kept = []
                for x in cands:
                    toks = range(x * bk, min(N, (x + 1) * bk)) if granularity == "block" else [x]
                    forced = any(t <= e and (t < sink or t >= r0 - local + 1) for t in toks)
                    if forced or best[x] >= 0:
                        kept.append(x)
                lists[b, g, i] = (kept, best)
    return lists


CASES = [
    # (B, N, Hq, Hkv, D, bq, bk, sink, local, gran)
    (1, 256, 1, 1, 16, 16, 16, 4, 16, "block"),
    (1, 250, 4, 1, 16, 32, 16, 4, 24, "block"),      # ragged N, GQA 4:1
    (2, 192, 4, 2, 16, 16, 16, 4, 20, "block"),      # batch 2, 2 groups
    (1, 200, 2, 1, 16, 32, 16, 4, 24, "stripe"),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("theta", [0.5, 1.2, 1.5, 1.8])
def test_bruteforce_matches_oracle(case, theta):
    B, N, Hq, Hkv, D, bq, bk, sink, local, gran = case
    rng = np.random.default_rng(hash((case, theta)) % (2 ** 32))
    q = bf16_values((B, N, Hq, D), rng)
    k = bf16_values((B, N, Hkv, D), rng)
    th = np.full(Hq, theta, dtype=np.float32)
    ref = brute_force_lists(q, k, th, bq=bq, bk=bk, sink=sink, local=local, granularity=gran)
    got = oracle.estimate_all(q, k, th, block_q=bq, block_k=bk, sink=sink, local=local,
                              granularity=gran)
    n_checked = 0
    for key, (kept, best) in ref.items():
        assert list(got[key]["kept"]) == kept, key
        np.testing.assert_allclose(got[key]["margin"], [best[x] for x in sorted(best)],
                                   rtol=0, atol=1e-9)
        n_checked += len(kept)
    assert n_checked > 0


def test_forced_sets_match_token_definition():
    N, bq, bk, sink, local = 1000, 64, 32, 32, 256
    for i in range(-(-N // bq)):
        r0, r1 = i * bq, min(N, (i + 1) * bq)
        want = sorted({t // bk for r in range(r0, r1) for t in range(r + 1)
                       if t < sink or t >= r - local + 1})
        assert list(oracle.forced_blocks(i, N, bq, bk, sink, local)) == want
        wantc = sorted({t for r in range(r0, r1) for t in range(r + 1)
                        if t < sink or t >= r - local + 1})
        assert list(oracle.forced_columns(i, N, bq, sink, local)) == wantc


def _small_inputs(seed=0, N=512, Hq=4, Hkv=2, D=32):
    rng = np.random.default_rng(seed)
    return bf16_values((1, N, Hq, D), rng), bf16_values((1, N, Hkv, D), rng)


KW = dict(block_q=64, block_k=32, sink=16, local=96)


def test_theta_nesting_forced_subset_and_extremes():
    q, k = _small_inputs()
    prev = None
    for th in [-np.inf, 0.5, 1.0, 1.5, 2.0, 3.0, np.inf]:
        r = oracle.estimate_all(q, k, np.full(4, th), **KW)
        for key, rec in r.items():
            assert set(rec["forced"]) <= set(rec["kept"])
            assert list(rec["kept"]) == sorted(set(rec["kept"]))
            if th == -np.inf:
                assert list(rec["kept"]) == list(rec["forced"])
            if th == np.inf:
                assert list(rec["kept"]) == list(range(rec["n_candidates"]))
            if prev is not None:
                assert set(prev[key]["kept"]) <= set(rec["kept"])
        prev = r


def test_union_contains_each_head_and_per_head_groups():
    q, k = _small_inputs(1)
    th = np.array([0.8, 1.4, 1.1, 2.0], dtype=np.float32)
    r = oracle.estimate_all(q, k, th, per_head=True, **KW)
    for rec in r.values():
        u = set()
        for kh in rec["kept_per_head"]:
            assert set(kh) <= set(rec["kept"])
            u |= set(kh)
        assert u == set(rec["kept"])
    # Hq == Hkv: each head on its own gives the same lists as the grouped call.
    q1, k1 = _small_inputs(2, Hq=2, Hkv=2)
    both = oracle.estimate_all(q1, k1, np.full(2, 1.2), **KW)
    for g in range(2):
        alone = oracle.estimate_all(q1[:, :, g:g + 1], k1[:, :, g:g + 1], np.full(1, 1.2), **KW)
        for (b, _, i), rec in alone.items():
            assert list(rec["kept"]) == list(both[(b, g, i)]["kept"])


def test_stripe_within_block():
    q, k = _small_inputs(3)
    for th in [0.8, 1.5]:
        blk = oracle.estimate_all(q, k, np.full(4, th), granularity="block", **KW)
        stp = oracle.estimate_all(q, k, np.full(4, th), granularity="stripe", **KW)
        for key in blk:
            cols = stp[key]["kept"]
            assert set(np.unique(cols // KW["block_k"])) <= set(blk[key]["kept"])


def test_key_shift_invariance_of_unquantised_margins():
    """Adding one vector u to every key moves x_a by c q_r.u, the pooled anchor by
    c qbar.u and every pooled score by c qbar.u, so margins are unchanged.  This holds only
    if anchor and query are pooled with the same (mean) weights."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 256, 2, 16))
    k = rng.standard_normal((1, 256, 1, 16))
    u = rng.standard_normal(16) * 3.0
    kw = dict(block_q=32, block_k=16, sink=8, local=40, quantized=False)
    a = oracle.estimate_all(q, k, np.full(2, 1.0), **kw)
    b = oracle.estimate_all(q, k + u, np.full(2, 1.0), **kw)
    for key in a:
        np.testing.assert_allclose(a[key]["margin"], b[key]["margin"], rtol=0, atol=1e-9)


def test_power_of_two_scale_invariance_is_bit_exact():
    q, k = _small_inputs(7)
    q2 = synth.bf16_round_bits(synth.bf16_bits_to_f32(q) * 4.0)
    for th in [0.7, 1.3]:
        a = oracle.estimate_all(q, k, np.full(4, th), **KW)
        b = oracle.estimate_all(q2, k, np.full(4, 4 * th), **KW)
        for key in a:
            assert list(a[key]["kept"]) == list(b[key]["kept"])
            np.testing.assert_array_equal(4 * a[key]["margin"], b[key]["margin"])


def test_quantizer_bounds_and_integer_dot():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((64, 128)) * rng.uniform(0.01, 10)).astype(np.float32)
    xq, s = oracle.quantize_q8(x, axis=None)
    assert xq.dtype == np.int8 and np.abs(xq.astype(int)).max() == 127
    err = np.abs(x.astype(np.float64) - float(s) * xq.astype(np.float64))
    assert err.max() <= float(s) / 2 * (1 + 1e-6)
    z, sz = oracle.quantize_q8(np.zeros(8, np.float32))
    assert float(sz) == 1.0 and not z.any()
    # integer dot products through the fp64 GEMM are exact
    a = rng.integers(-127, 128, (8, 128))
    b = rng.integers(-127, 128, (128, 16))
    got = a.astype(np.float64) @ b.astype(np.float64)
    for i in range(8):
        for j in range(16):
            assert got[i, j] == sum(int(a[i, t]) * int(b[t, j]) for t in range(128))


def test_tiny_workload_density_sweep():
    """The tiny 4K workload: theta 4.0 keeps every causal block (the Jensen gap between the
    row-max anchor and pooled scores), -inf keeps exactly the forced blocks."""
    x = synth.make_prefill("tiny_4k")
    kw = dict(block_q=64, block_k=64, sink=32, local=256)
    full = oracle.estimate_all(x.q, x.k, x.theta, **kw)
    assert all(len(r["kept"]) == r["n_candidates"] for r in full.values())
    low = oracle.estimate_all(x.q, x.k, np.full(1, -np.inf), **kw)
    assert all(list(r["kept"]) == list(r["forced"]) for r in low.values())
    mid = oracle.estimate_all(x.q, x.k, np.full(1, 2.5), **kw)
    dens = sum(len(r["kept"]) for r in mid.values()) / sum(r["n_candidates"] for r in mid.values())
    assert 0.2 < dens < 0.9
