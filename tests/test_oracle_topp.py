"""Pins of the oracle's top-p decode budget (CPU).

The budget is the fewest content blocks that bring the forced share plus theirs of
pi = softmax(block scores) to at least top_p (the reading of SpotAttention's top-p rule).
Pinned against: a brute force over every subset of content blocks (the smallest subset
size whose best mass reaches the target), closed forms for uniform and two-level scores,
invariance under a common shift of the scores, monotonicity in top_p, and the cap at K
through decode_select.
"""
import itertools

import numpy as np
import pytest

import oracle
from oracle.decode import TOP_P_BAND, top_p_budget


def _brute_budget(score, is_forced, p):
    w = np.exp(score - score.max())
    z = w.sum()
    base = w[is_forced].sum() / z
    rest = np.nonzero(~is_forced)[0]
    for size in range(rest.size + 1):
        best = max((w[list(c)].sum() for c in itertools.combinations(rest, size)), default=0.0)
        if base + best / z >= p:
            return size
    return rest.size


@pytest.mark.parametrize("seed", range(12))
def test_budget_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(3, 10))
    score = rng.normal(0.0, 1.5, n)
    is_f = np.zeros(n, dtype=bool)
    is_f[rng.choice(n, size=int(rng.integers(0, 3)), replace=False)] = True
    for p in [0.1, 0.3, 0.5, 0.7, 0.9, 0.97]:
        k, order, amb = top_p_budget(score, is_f, p)
        if not amb:
            assert k == _brute_budget(score, is_f, p), (seed, p)
        # the chosen blocks are the highest-scoring content blocks
        assert sorted(score[order[:k]].tolist(), reverse=True) == \
            sorted(score[~is_f].tolist(), reverse=True)[:k]


def test_uniform_scores_closed_form():
    n, nf = 40, 3
    is_f = np.zeros(n, dtype=bool)
    is_f[:nf] = True
    for p in [0.06, 0.33, 0.51, 0.77, 0.99]:         # p * n never an integer
        k, _, amb = top_p_budget(np.full(n, 0.7), is_f, p)
        assert not amb
        assert k == max(0, int(np.ceil(p * n - 1e-12)) - nf)


def test_two_level_closed_form():
    # one block at score a, the other n-1 at 0: its share is e^a / (e^a + n - 1)
    n, a = 20, 3.0
    score = np.zeros(n)
    score[7] = a
    share = np.exp(a) / (np.exp(a) + n - 1)
    is_f = np.zeros(n, dtype=bool)
    k, order, _ = top_p_budget(score, is_f, share - 0.01)
    assert k == 1 and order[0] == 7
    k, _, _ = top_p_budget(score, is_f, share + 0.01)
    rest = (share + 0.01 - share) * (np.exp(a) + n - 1)      # mass still needed, unit blocks
    assert k == 1 + int(np.ceil(rest))


def test_shift_invariance_and_monotone():
    rng = np.random.default_rng(5)
    score = rng.normal(0, 2, 300)
    is_f = np.zeros(300, dtype=bool)
    is_f[[0, 297, 298, 299]] = True
    prev = 0
    for p in np.linspace(0.01, 0.999, 40):
        k, _, amb = top_p_budget(score, is_f, p)
        k2, _, amb2 = top_p_budget(score + 123.25, is_f, p)
        if not (amb or amb2):
            assert k == k2
        assert k >= prev
        prev = k


def test_forced_share_enough_and_full():
    score = np.array([5.0, -3.0, -3.0, -3.0, 5.0])
    is_f = np.array([True, False, False, False, True])
    k, _, _ = top_p_budget(score, is_f, 0.9)                 # forced hold > 0.99 of the mass
    assert k == 0
    k, _, _ = top_p_budget(score, is_f, 1.0)
    assert k == 3


def test_decode_select_caps_at_k_and_keeps_forced():
    rng = np.random.default_rng(9)
    B, Hq, Hkv, D, L, bk = 1, 4, 1, 64, 64 * 40, 64
    q = rng.normal(size=(B, Hq, D)).astype(np.float32)
    kbar = rng.normal(size=(B, 40, Hkv, D)).astype(np.float32)
    for top_k, p in [(8, 0.999), (40, 0.999), (40, 0.2)]:
        sel = oracle.decode_select(q, kbar, np.array([L]), block_k=bk, top_k=top_k, sink=32,
                                   local=256, top_p=p)[(0, 0)]
        f = set(sel["forced"].tolist())
        assert f <= set(sel["selected"].tolist())
        assert len(sel["selected"]) == len(f) + sel["budget"] <= max(top_k, len(f))
        assert sel["budget"] == min(sel["budget_uncapped"], top_k - len(f))
    # p = 0.999 over 40 near-uniform blocks needs almost every block: the cap of 8 binds
    sel = oracle.decode_select(q, kbar, np.array([L]), block_k=bk, top_k=8, sink=32, local=256,
                               top_p=0.999)[(0, 0)]
    assert len(sel["selected"]) == 8


def test_band_flags_exact_boundary():
    score = np.zeros(10)
    k, _, amb = top_p_budget(score, np.zeros(10, dtype=bool), 0.5 + TOP_P_BAND / 2)
    assert amb and k == 6
