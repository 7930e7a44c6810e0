"""Pins of the oracle's grouped identification (AnchorAttention's step) (CPU).

Brute force: for every block the kept set is recomputed from the group's per-block threshold
results by plain set operations written out here differently (a loop over every candidate
of every block); plus the invariants the reading fixes: step = 1 is the identity; grouping
only adds entries; every block of a group holds the same non-forced entries on its causal
range; groups nest (step 2 within step 4 within step 8 for aligned groups); the last group
may be partial.
"""
import numpy as np
import pytest

import oracle
import synth


@pytest.fixture(scope="module")
def base():
    x = synth.make_prefill("llama8b_32k", seq=3000, hq=8, hkv=2)
    theta = np.repeat(np.array([3.0, 6.0], np.float32), 4)
    ref = oracle.estimate_all(x.q, x.k, theta, block_q=128, block_k=64, sink=32, local=256)
    return ref


def test_identity_at_step_one(base):
    assert oracle.group_step(base, 1) is base


@pytest.mark.parametrize("step", [2, 3, 4, 16])
def test_brute_force(base, step):
    got = oracle.group_step(base, step)
    for (b, g, i), r in base.items():
        nc = r["n_candidates"]
        want = []
        for J in range(nc):
            keep = J in set(r["forced"].tolist())
            for i2 in range((i // step) * step, (i // step + 1) * step):
                r2 = base.get((b, g, i2))
                if r2 is not None and J < r2["margin"].size and r2["margin"][J] >= 0:
                    keep = True
            if keep:
                want.append(J)
        assert got[(b, g, i)]["kept"].tolist() == want


@pytest.mark.parametrize("step", [2, 4, 16])
def test_invariants(base, step):
    got = oracle.group_step(base, step)
    for key, r in base.items():
        assert set(r["kept"].tolist()) <= set(got[key]["kept"].tolist())
    nqb = max(i for (_, _, i) in base) + 1
    for (b, g, i), r in got.items():
        i0 = (i // step) * step
        first = got[(b, g, i0)]
        nc0 = first["n_candidates"]
        mine = set(r["kept"].tolist()) - set(r["forced"].tolist())
        theirs = set(first["kept"].tolist()) - set(first["forced"].tolist())
        # on the first block's causal range the non-forced entries agree (forced sets differ)
        fr = set(r["forced"].tolist()) | set(first["forced"].tolist())
        assert {J for J in mine if J < nc0} - fr == {J for J in theirs} - fr
    assert nqb == 24


def test_groups_nest(base):
    s2, s4, s8 = (oracle.group_step(base, s) for s in (2, 4, 8))
    for key in base:
        assert set(s2[key]["kept"].tolist()) <= set(s4[key]["kept"].tolist()) <= \
            set(s8[key]["kept"].tolist())
