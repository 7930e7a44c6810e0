"""Pins of the oracle's MXFP4 quantiser (OCP Microscaling Formats v1.0: per 32 elements a
shared scale 2^e, e = floor(log2(max|x|)) - 2, elements E2M1 with round-to-nearest-even and
saturation at 6) (CPU).

Pinned against: exact round trip of representable values, the E2M1 tie cases worked out from
the grid {0, 0.5, 1, 1.5, 2, 3, 4, 6} (ties go to the code with mantissa bit 0), the scale rule
on random blocks, the error bound, sign symmetry, and the all-zero block.
"""
import numpy as np
import pytest

from oracle.estimate_sale import E2M1_GRID, dequantize_mxfp4, quantize_mxfp4


def test_representable_round_trip():
    rng = np.random.default_rng(0)
    for _ in range(50):
        e = int(rng.integers(-20, 20))
        v = rng.choice(np.concatenate([E2M1_GRID, -E2M1_GRID]), size=(3, 64))
        v[:, ::32] = 6.0                                  # every block reaches the top code
        x = (v * 2.0 ** e).astype(np.float32)
        vals, exps = quantize_mxfp4(x)
        assert np.all(exps == e)
        assert np.array_equal(dequantize_mxfp4(vals, exps), x.astype(np.float64))


def test_ties_and_saturation():
    y = np.zeros((1, 32), np.float32)
    y[0, :9] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -2.5]
    y[0, 31] = 7.5                                        # max 7.5 -> e = floor(log2 7.5) - 2 = 0
    vals, exps = quantize_mxfp4(y)
    assert exps[0, 0] == 0
    # 0.25 -> 0 (0 even), 0.75 -> 1 (1.0 even), 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4,
    # 7 and 7.5 saturate to 6
    assert vals[0, :9].tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, -2.0]
    assert vals[0, 31] == 6.0


@pytest.mark.parametrize("seed", range(5))
def test_scale_rule_error_bound_symmetry(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((40, 128)) * np.exp(rng.uniform(-8, 8, (40, 1)))).astype(np.float32)
    vals, exps = quantize_mxfp4(x)
    blocks = np.abs(x.astype(np.float64)).reshape(40, 4, 32).max(axis=-1)
    k = np.floor(np.log2(blocks))
    assert np.array_equal(exps, (k - 2).astype(np.int64))
    assert np.all(2.0 ** k <= blocks) and np.all(blocks < 2.0 ** (k + 1))
    q = dequantize_mxfp4(vals, exps)
    step = np.repeat(np.ldexp(1.0, exps), 32, axis=-1)
    err = np.abs(q - x.astype(np.float64))
    y = np.abs(x.astype(np.float64)) / step
    assert np.all(err[y <= 6] <= step[y <= 6] + 0.0)       # half of the widest spacing (2)
    assert np.all(err <= 2 * step)                        # saturation region (6, 8)
    vn, en = quantize_mxfp4(-x)
    assert np.array_equal(vn, -vals) and np.array_equal(en, exps)


def test_zero_block():
    vals, exps = quantize_mxfp4(np.zeros((2, 64), np.float32))
    assert np.all(vals == 0) and np.all(exps == -127)
