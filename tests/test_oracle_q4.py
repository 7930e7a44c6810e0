"""Pins of the oracle's 4-bit block-summary quantiser (CPU only).

Closed-form cases (a group's max maps to +-7, zero groups, round-half-to-even ties), the
rounding-error bound of the scheme, and an independent unpacking of the packed nibbles."""
import numpy as np

import oracle
import synth


def _bits(x):
    return synth.bf16_round_bits(np.asarray(x, dtype=np.float32))


def test_extremes_zero_and_ties():
    x = np.zeros((2, 32), dtype=np.float32)
    x[0, 0], x[0, 1], x[0, 2] = 7.0, -7.0, 2.5       # scale 1: codes 7, -7, and the tie 2.5 -> 2
    x[0, 3], x[0, 4] = 3.5, -0.5                     # ties to even: 4, -0
    codes, scales = oracle.quantize_summary_q4(_bits(x))
    assert codes[0, :5].tolist() == [7, -7, 2, 4, 0]
    assert np.all(codes[1] == 0) and scales[1] == 0          # an all-zero group
    assert synth.bf16_bits_to_f64(scales[0:1])[0] == 1.0


def test_error_bound_and_range():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 128)).astype(np.float32) * rng.uniform(0.01, 10, (64, 1)).astype(np.float32)
    kb = _bits(x)
    codes, scales = oracle.quantize_summary_q4(kb)
    assert codes.min() >= -7 and codes.max() <= 7
    xv = synth.bf16_bits_to_f64(kb).reshape(64, 4, 32)
    a = np.abs(xv).max(axis=-1)
    c = codes.reshape(64, 4, 32)
    assert np.all(np.abs(c).max(axis=-1) == 7)               # every group's max reaches 7
    deq = oracle.dequantize_summary_q4(codes, scales).reshape(64, 4, 32)
    # half a quantisation step plus the bf16 rounding of the scale (<= 2^-9 relative) at 7 steps
    bound = a / 7 * 0.5 * (1 + 1e-6) + 7 * (a / 7) * 2.0 ** -8
    assert np.all(np.abs(deq - xv) <= bound[..., None])


def test_packing():
    rng = np.random.default_rng(1)
    codes = rng.integers(-7, 8, size=(3, 5, 2, 64)).astype(np.int8)
    packed = oracle.pack_q4(codes)
    assert packed.shape == (3, 5, 2, 32) and packed.dtype == np.uint8
    flat_p, flat_c = packed.reshape(-1, 4), codes.reshape(-1, 8)
    for i in range(flat_p.shape[0]):
        word = int.from_bytes(bytes(flat_p[i].tolist()), "little")
        for d in range(8):
            nib = d // 2 + (4 if d % 2 else 0)            # dim 2j -> nibble j, 2j+1 -> j+4
            assert ((word >> (4 * nib)) & 0xF) - 8 == flat_c[i, d]
