"""Pins of the FP4 (MXFP4) block-summary oracle (CPU).

SpotAttention "Key findings": the selector's key cache in INT4 or FP4 microscale.  The FP4
form here is OCP Microscaling v1.0 MXFP4; these tests decode the packed storage with the
format's own bit-field definition of E2M1 (sign, two exponent bits with bias 1, one mantissa
bit; exponent field 0 is subnormal) and of E8M0 (2^(byte - 127)), independently of the
oracle's grid table."""
import numpy as np

import oracle
from oracle.decode import _f32_to_bf16_bits


def _bits(x):
    return _f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _e2m1_from_fields(n):
    """E2M1 nibble -> value from its bit fields."""
    s = -1.0 if n & 8 else 1.0
    e, m = (n >> 1) & 3, n & 1
    if e == 0:
        return s * 0.5 * m                       # subnormal: m * 2^(1 - bias) * 0.5
    return s * 2.0 ** (e - 1) * (1.0 + 0.5 * m)


def _decode_storage(codes, exps):
    """codes uint8 [..., D/2], exps uint8 [..., D/32] -> float64 [..., D]."""
    lo = np.vectorize(_e2m1_from_fields)(codes & 15)
    hi = np.vectorize(_e2m1_from_fields)(codes >> 4)
    vals = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,))
    vals[..., 0::2], vals[..., 1::2] = lo, hi
    scale = np.repeat(2.0 ** (exps.astype(np.float64) - 127.0), 32, axis=-1)
    return vals * scale


def _summaries(seed, shape=(3, 5, 2, 128)):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape) * np.exp(rng.uniform(-6, 3, shape[:-1] + (1,)))
    return _bits(x)


def test_storage_decodes_to_the_oracle_values():
    kb = _summaries(0)
    vals, exps = oracle.quantize_summary_fp4(kb)
    codes, eb = oracle.pack_fp4(kb, vals, exps)
    assert codes.shape == kb.shape[:-1] + (64,) and eb.shape == kb.shape[:-1] + (4,)
    np.testing.assert_array_equal(_decode_storage(codes, eb),
                                  oracle.dequantize_summary_fp4(vals, exps))


def test_scale_rule_and_error_bound():
    kb = _summaries(1)
    x = oracle.decode._f64(kb)
    vals, exps = oracle.quantize_summary_fp4(kb)
    deq = oracle.dequantize_summary_fp4(vals, exps)
    g = x.reshape(x.shape[:-1] + (4, 32))
    amax = np.abs(g).max(axis=-1)
    # the largest magnitude of a group lands in [4, 8) * 2^e, so it is stored as 4 or 6 * 2^e
    assert np.all((amax >= 4.0 * 2.0 ** exps) & (amax < 8.0 * 2.0 ** exps))
    err = np.abs(deq - x).reshape(g.shape)
    step = 2.0 ** exps[..., None]
    # below 6 * 2^e the grid spacing is at most 2 * 2^e: nearest rounding is within half of it;
    # above, saturation at 6 * 2^e costs less than 2 * 2^e
    assert np.all(err <= step * np.where(np.abs(g) <= 6 * step, 1.0, 2.0))
    # saturation only ever lowers a magnitude
    big = np.abs(g) > 6 * step
    assert np.all(np.abs(deq.reshape(g.shape))[big] == 6 * np.broadcast_to(step, g.shape)[big])


def test_exact_values_round_trip_and_signs():
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    row = np.concatenate([grid, -grid, grid[::-1], -grid[::-1]]) * 2.0 ** -3     # 32 dims
    x = np.concatenate([row, row * 4.0, row * 2.0 ** 20, np.zeros(32)])[None, :]
    kb = _bits(x)
    vals, exps = oracle.quantize_summary_fp4(kb)
    np.testing.assert_array_equal(oracle.dequantize_summary_fp4(vals, exps), x)
    codes, eb = oracle.pack_fp4(kb, vals, exps)
    assert eb[0, 3] == 0                        # all-zero group: exponent -127
    # group maxima 0.75, 3 and 6 * 2^17: e = floor(log2 max) - 2 = -3, -1, 17
    assert list(eb[0, :3]) == [124, 126, 144]
    # negative zero keeps its sign bit (nibble 8); 1.0 in a group of max 1 (e = -2) is 4 * 2^e,
    # magnitude index 6
    nz = _bits(np.array([[-0.0] + [1.0] * 31]))
    c, _ = oracle.pack_fp4(nz, *oracle.quantize_summary_fp4(nz))
    assert c[0, 0] == 0x68 and c[0, 1] == 0x66


def test_ties_go_to_the_even_code():
    # midpoints between grid neighbours, at e = 0 (the group max 4 fixes e = floor(log2 4) - 2)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    want = np.array([0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0])
    x = np.concatenate([mids, [4.0], np.zeros(24)])[None, :]
    vals, exps = oracle.quantize_summary_fp4(_bits(x))
    assert exps[0, 0] == 0
    np.testing.assert_array_equal(vals[0, :7], want)


def test_fp4_scores_are_dot_products_with_the_decoded_storage():
    # decode selection from FP4 summaries scores with exactly the decoded storage values
    rng = np.random.default_rng(3)
    B, L, Hkv, Hq, D, bk = 2, 700, 2, 4, 64, 64
    k = _bits(rng.standard_normal((B, L, Hkv, D)))
    q = _bits(rng.standard_normal((B, Hq, D)))
    lens = np.array([700, 333])
    kbar = oracle.block_summary(k, lens, bk)
    vals, exps = oracle.quantize_summary_fp4(kbar)
    codes, eb = oracle.pack_fp4(kbar, vals, exps)
    dec = _decode_storage(codes, eb)
    sel = oracle.decode_select(q, oracle.dequantize_summary_fp4(vals, exps), lens, block_k=bk,
                               top_k=4, sink=32, local=64)
    c = 1.0 / np.sqrt(D)
    for b in range(B):
        nkb = -(-int(lens[b]) // bk)
        for g in range(Hkv):
            qh = oracle.decode._f64(q[b, 2 * g:2 * g + 2])
            brute = np.array([max(c * float(qh[h] @ dec[b, J, g]) for h in range(2))
                              for J in range(nkb)])
            np.testing.assert_allclose(sel[(b, g)]["score"], brute, rtol=1e-12, atol=1e-12)
