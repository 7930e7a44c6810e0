"""The tiny 4K workload is fp32 on the pages' list of configurations; the GPU path and the
oracle both consume it rounded once to bf16.  Self-check of that rounding: the oracle run on
the fp32 originals and on the bf16-rounded values must agree on the kept lists (outside the
ambiguity band of either run) and on the attention output within the bars the GPU is held to,
so the rounding of the fp32 inputs is not what the parity tolerances absorb.  fp32 inputs
are carried in float64 by the oracle (every fp32 value is exact in fp64)."""
import numpy as np

import oracle
import synth

KW = dict(block_q=64, block_k=64, sink=32, local=256)


def _both(theta):
    x = synth.make_prefill("tiny_4k")
    assert x.f32 is not None
    th = np.full(1, theta, np.float32)
    ref16 = oracle.estimate_all(x.q, x.k, th, **KW)
    ref32 = oracle.estimate_all(x.f32["q"], x.f32["k"], th, **KW)
    return x, ref16, ref32


def test_fp32_originals_give_the_same_lists_and_output():
    for theta in [4.0, 2.5, 2.0, 1.5]:
        x, ref16, ref32 = _both(theta)
        flips = 0
        for key in ref16:
            a, b = set(ref16[key]["kept"].tolist()), set(ref32[key]["kept"].tolist())
            amb = set(ref16[key]["ambiguous"].tolist()) | set(ref32[key]["ambiguous"].tolist())
            # a decision can move with the input rounding only where the margin is small
            m16 = ref16[key]["margin"]
            for J in a ^ b:
                assert J in amb or abs(m16[J]) < 0.05, (theta, key, J, m16[J])
            flips += len(a ^ b)
        lists = {key: r["kept"] for key, r in ref16.items()}
        O16, L16 = oracle.attention_all(x.q, x.k, x.v, lists, **{k: KW[k] for k in ("block_q", "block_k")})
        O32, L32 = oracle.attention_all(x.f32["q"], x.f32["k"], x.f32["v"], lists,
                                        **{k: KW[k] for k in ("block_q", "block_k")})
        err = np.abs(O16 - O32)
        assert err.max() < 2e-2 and err.mean() < 2e-3, (theta, err.max(), err.mean())
        assert np.abs(L16 - L32).max() < 1e-2
        # and the rounding is visible (the fp32 run really used the originals)
        assert err.max() > 0.0


def test_fp32_originals_round_to_the_bf16_inputs():
    x = synth.make_prefill("tiny_4k")
    for name in ("q", "k", "v"):
        f = np.asarray(x.f32[name], np.float32)
        bits = getattr(x, name)
        # round to nearest even of the fp32 bits, written out from the bf16 definition
        u = f.view(np.uint32).astype(np.uint64)
        r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
        np.testing.assert_array_equal(r, bits)
