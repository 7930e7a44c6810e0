"""Named workloads and their seeded generators.

Every tensor is drawn in float32 from numpy's PCG64 streams, derived with
``SeedSequence(seed).spawn`` in a fixed order (Q, K, V, needle positions, needle
queries, theta), and rounded once to bfloat16 (round to nearest even).  The oracle and
the GPU path consume the same bfloat16 values, passed around as uint16 bit patterns.

Workload recipe (synthetic stand-ins for the long-context retrieval suites the pages
evaluate on; no item of any suite is reproduced):

* Q, K, V ~ N(0, 1), layout ``[batch, seq, heads, head_dim]``.
* Llama-3.1-8B-shaped workloads add a rank-16 rotary-style positional term to dims
  0..15 of Q and K: ``alpha * [cos(t w_m), sin(t w_m)]`` with ``w_m = 500000 **
  (-2 k_m / 128)`` for ``k_m in {16, 22, ..., 58}`` and ``alpha = 3``.  Its low
  frequencies make the sink shift below a real bias and give the scores a diagonal
  (local) band.
* Attention sink: keys 0..31 of every KV head get ``+4 * mean(Q)``, the mean taken over
  tokens and over the query heads sharing that KV head.
* Needles: a fraction of key positions (uniform, or in the middle half of the context)
  are overwritten with ``3 * q_r / |q_r|`` for a random later query row ``r`` of a random
  query head in the group.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# --------------------------------------------------------------------------------------
# Workloads.  Sizes follow the configurations the sparse-prefill and sparse-decode pages
# are evaluated at (Llama-3.1-8B attention: 32 query / 8 KV heads, head_dim 128).
# --------------------------------------------------------------------------------------
CONFIGS: dict[str, dict] = {
    # Tiny single-head case: the oracle finishes it in seconds.
    "tiny_4k": dict(kind="prefill", batch=1, hq=1, hkv=1, seq=4096, head_dim=64,
                    dtype="fp32", block_q=64, block_k=64, sink=32, local=256,
                    granularity="block", theta=4.0, positional=False,
                    needle_count=16, needle_region="any"),
    # One Llama-3.1-8B-shaped attention layer at 32K.
    "llama8b_32k": dict(kind="prefill", batch=1, hq=32, hkv=8, seq=32768, head_dim=128,
                        dtype="bf16", block_q=128, block_k=64, sink=32, local=256,
                        granularity="block", theta=4.0, positional=True,
                        needle_frac=0.01, needle_region="any"),
    # The same layer at 128K with a per-KV-head threshold from {2, 3, 4, 6}.
    "llama8b_128k": dict(kind="prefill", batch=1, hq=32, hkv=8, seq=131072, head_dim=128,
                         dtype="bf16", block_q=128, block_k=64, sink=32, local=256,
                         granularity="block", theta="per_kv_head", theta_choices=(2.0, 3.0, 4.0, 6.0),
                         positional=True, needle_frac=0.01, needle_region="any"),
    # Stripe granularity (query block x single key column) at 64K.
    "stripe_64k": dict(kind="prefill", batch=1, hq=32, hkv=8, seq=65536, head_dim=128,
                       dtype="bf16", block_q=128, block_k=64, sink=32, local=256,
                       granularity="stripe", theta=3.0, positional=True,
                       needle_frac=0.005, needle_region="middle"),
    # Batched single-token decode over a 128K cache.
    "decode_b16_128k": dict(kind="decode", batch=16, hq=32, hkv=8, seq=131072, head_dim=128,
                            dtype="bf16", block_k=64, top_k=64, sink=32, local=256,
                            positional=True, needle_frac=0.01, needle_region="any"),
}

POS_ALPHA = 3.0
POS_BASE = 500000.0
POS_K = tuple(range(16, 64, 6))   # 16, 22, ..., 58  -> 8 frequencies, 16 dims
SINK_TOKENS_SHIFTED = 32
SINK_GAIN = 4.0
NEEDLE_GAIN = 3.0


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# --------------------------------------------------------------------------------------
# bfloat16 helpers (bit manipulation only).
# --------------------------------------------------------------------------------------
def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bfloat16 bit patterns, round to nearest even (finite input)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_u.size, step):
        c = flat_u[s:s + step].astype(np.uint64)
        c = (c + 0x7FFF + ((c >> 16) & 1)) >> 16
        flat_o[s:s + step] = c.astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


# --------------------------------------------------------------------------------------
# Containers.
# --------------------------------------------------------------------------------------
@dataclass
class PrefillInputs:
    name: str
    seed: int
    q: np.ndarray            # uint16 bf16 bits [B, N, Hq, d]
    k: np.ndarray            # uint16 bf16 bits [B, N, Hkv, d]
    v: np.ndarray            # uint16 bf16 bits [B, N, Hkv, d]
    theta: np.ndarray        # float32 [Hq], logit units
    block_q: int
    block_k: int
    sink: int
    local: int
    granularity: str         # "block" | "stripe"
    needles: list = field(default_factory=list)   # per (b, g): sorted needle positions
    f32: dict | None = None  # fp32 originals (tiny fp32 workload only)

    @property
    def shape(self):
        b, n, hq, d = self.q.shape
        return dict(batch=b, seq=n, hq=hq, hkv=self.k.shape[2], head_dim=d)


@dataclass
class DecodeInputs:
    name: str
    seed: int
    q: np.ndarray            # uint16 bf16 bits [B, Hq, d], the query at position L-1
    k_cache: np.ndarray      # uint16 bf16 bits [B, L, Hkv, d]
    v_cache: np.ndarray      # uint16 bf16 bits [B, L, Hkv, d]
    cache_len: np.ndarray    # int32 [B]
    block_k: int
    top_k: int
    sink: int
    local: int


# --------------------------------------------------------------------------------------
# Building blocks.
# --------------------------------------------------------------------------------------
def _fill_normal(out: np.ndarray, ss: np.random.SeedSequence, pool: ThreadPoolExecutor) -> None:
    """out[b, :, h, :] <- N(0,1) from one child stream per (b, h)."""
    B, _, H, _ = out.shape
    kids = ss.spawn(B * H)

    def work(idx):
        b, h = divmod(idx, H)
        g = np.random.Generator(np.random.PCG64(kids[idx]))
        out[b, :, h, :] = g.standard_normal((out.shape[1], out.shape[3]), dtype=np.float32)

    list(pool.map(work, range(B * H)))


def positional_term(t: np.ndarray) -> np.ndarray:
    """[len(t), 16] float64 rotary-style term for positions t (dims 2m, 2m+1 = cos, sin)."""
    t = np.asarray(t, dtype=np.float64)[:, None]
    w = POS_BASE ** (-2.0 * np.asarray(POS_K, dtype=np.float64) / 128.0)[None, :]
    p = np.empty((t.shape[0], 2 * len(POS_K)), dtype=np.float64)
    p[:, 0::2] = POS_ALPHA * np.cos(t * w)
    p[:, 1::2] = POS_ALPHA * np.sin(t * w)
    return p


def _add_positional(x: np.ndarray, pool: ThreadPoolExecutor) -> None:
    B, N, H, _ = x.shape
    step = 8192

    def work(s):
        p = positional_term(np.arange(s, min(N, s + step))).astype(np.float32)
        x[:, s:s + step, :, 0:16] += p[None, :, None, :]

    list(pool.map(work, range(0, N, step)))


def _needle_positions(rng, n_keys: int, count: int, region: str) -> np.ndarray:
    if region == "middle":
        lo, hi = n_keys // 4, (3 * n_keys) // 4
    else:
        lo, hi = SINK_TOKENS_SHIFTED, n_keys - 1
    count = min(count, max(0, hi - lo))
    return np.sort(rng.choice(np.arange(lo, hi), size=count, replace=False))


# --------------------------------------------------------------------------------------
# Prefill generator.
# --------------------------------------------------------------------------------------
def make_prefill(name: str, seed: int = 0, *, seq: int | None = None, batch: int | None = None,
                 hq: int | None = None, hkv: int | None = None, head_dim: int | None = None,
                 theta=None) -> PrefillInputs:
    """Generate one prefill workload.  Keyword overrides shrink it for fast tests
    while keeping the recipe (positional term, sink shift, needle density)."""
    cfg = dict(CONFIGS[name])
    assert cfg["kind"] == "prefill", name
    B = batch or cfg["batch"]
    N = seq or cfg["seq"]
    Hq = hq or cfg["hq"]
    Hkv = hkv or cfg["hkv"]
    D = head_dim or cfg["head_dim"]
    assert Hq % Hkv == 0
    grp = Hq // Hkv
    ss = np.random.SeedSequence(seed)
    s_q, s_k, s_v, s_pos, s_nq, s_theta = ss.spawn(6)
    q = np.empty((B, N, Hq, D), dtype=np.float32)
    k = np.empty((B, N, Hkv, D), dtype=np.float32)
    v = np.empty((B, N, Hkv, D), dtype=np.float32)
    with ThreadPoolExecutor(_threads()) as pool:
        _fill_normal(q, s_q, pool)
        _fill_normal(k, s_k, pool)
        _fill_normal(v, s_v, pool)
        if cfg["positional"] and D >= 16:
            _add_positional(q, pool)
            _add_positional(k, pool)
    # Sink shift on the first keys: +4 * mean over tokens and the group's query heads.
    n_sink = min(SINK_TOKENS_SHIFTED, N)
    for b in range(B):
        for g in range(Hkv):
            mu = q[b, :, g * grp:(g + 1) * grp, :].astype(np.float64).mean(axis=(0, 1))
            k[b, :n_sink, g, :] += (SINK_GAIN * mu).astype(np.float32)[None, :]
    # Needles.
    pos_kids = s_pos.spawn(B * Hkv)
    nq_kids = s_nq.spawn(B * Hkv)
    needles = []
    for b in range(B):
        for g in range(Hkv):
            rp = np.random.Generator(np.random.PCG64(pos_kids[b * Hkv + g]))
            rq = np.random.Generator(np.random.PCG64(nq_kids[b * Hkv + g]))
            if "needle_count" in cfg:
                count = cfg["needle_count"]
            else:
                count = int(round(cfg["needle_frac"] * N))
            pos = _needle_positions(rp, N, count, cfg["needle_region"])
            for p in pos:
                r = int(rq.integers(p + 1, N))
                h = g * grp + int(rq.integers(0, grp))
                qr = q[b, r, h, :].astype(np.float64)
                k[b, p, g, :] = (NEEDLE_GAIN * qr / np.linalg.norm(qr)).astype(np.float32)
            needles.append(pos)
    # Threshold per query head.
    if theta is not None:
        th = np.broadcast_to(np.asarray(theta, dtype=np.float32), (Hq,)).copy()
    elif cfg["theta"] == "per_kv_head":
        rt = np.random.Generator(np.random.PCG64(s_theta))
        tg = rt.choice(np.asarray(cfg["theta_choices"], dtype=np.float32), size=Hkv)
        th = np.repeat(tg, grp).astype(np.float32)
    else:
        th = np.full((Hq,), cfg["theta"], dtype=np.float32)
    f32 = None
    if cfg["dtype"] == "fp32":
        f32 = dict(q=q.copy(), k=k.copy(), v=v.copy())
    out = PrefillInputs(name=name, seed=seed, q=bf16_round_bits(q), k=bf16_round_bits(k),
                        v=bf16_round_bits(v), theta=th, block_q=cfg["block_q"],
                        block_k=cfg["block_k"], sink=cfg["sink"], local=cfg["local"],
                        granularity=cfg["granularity"], needles=needles, f32=f32)
    return out


# --------------------------------------------------------------------------------------
# Decode generator.
# --------------------------------------------------------------------------------------
def make_decode(name: str = "decode_b16_128k", seed: int = 0, *, batch: int | None = None,
                seq: int | None = None, hq: int | None = None, hkv: int | None = None,
                head_dim: int | None = None, top_k: int | None = None) -> DecodeInputs:
    """Batched decode workload: B independent caches of L tokens and one query per
    sequence at position L-1.  The query matrix of the prefill recipe is not
    materialised: the sink shift uses the positional mean plus a draw of the noise
    mean with its exact N(0, 1/(L*group)) law, and needle directions are fresh query
    rows drawn at their positions."""
    cfg = dict(CONFIGS[name])
    assert cfg["kind"] == "decode", name
    B = batch or cfg["batch"]
    L = seq or cfg["seq"]
    Hq = hq or cfg["hq"]
    Hkv = hkv or cfg["hkv"]
    D = head_dim or cfg["head_dim"]
    grp = Hq // Hkv
    kq = np.empty((B, Hq, D), dtype=np.float32)
    kc = np.empty((B, L, Hkv, D), dtype=np.uint16)
    vc = np.empty((B, L, Hkv, D), dtype=np.uint16)
    seq_kids = np.random.SeedSequence(seed).spawn(B)
    with ThreadPoolExecutor(_threads()) as pool:
        for b in range(B):
            s_q, s_k, s_v, s_pos, s_nq, _ = seq_kids[b].spawn(6)
            k = np.empty((1, L, Hkv, D), dtype=np.float32)
            v = np.empty((1, L, Hkv, D), dtype=np.float32)
            _fill_normal(k, s_k, pool)
            _fill_normal(v, s_v, pool)
            pmean = np.zeros(D)
            if cfg["positional"] and D >= 16:
                _add_positional(k, pool)
                pmean[:16] = positional_term(np.arange(L)).mean(axis=0)
            rq = np.random.Generator(np.random.PCG64(s_q))
            qrow = rq.standard_normal((Hq, D)).astype(np.float32)
            if cfg["positional"] and D >= 16:
                qrow[:, :16] += positional_term(np.array([L - 1]))[0].astype(np.float32)
            kq[b] = qrow
            n_sink = min(SINK_TOKENS_SHIFTED, L)
            rn = np.random.Generator(np.random.PCG64(s_nq))
            pos_kids = s_pos.spawn(Hkv)
            for g in range(Hkv):
                mu = pmean + rn.standard_normal(D) / np.sqrt(L * grp)
                k[0, :n_sink, g, :] += (SINK_GAIN * mu).astype(np.float32)[None, :]
                rp = np.random.Generator(np.random.PCG64(pos_kids[g]))
                pos = _needle_positions(rp, L, int(round(cfg["needle_frac"] * L)),
                                        cfg["needle_region"])
                rows = rn.integers(pos + 1, L) if len(pos) else np.zeros(0, dtype=np.int64)
                dirs = rn.standard_normal((len(pos), D))
                if cfg["positional"] and D >= 16:
                    dirs[:, :16] += positional_term(rows)
                dirs /= np.linalg.norm(dirs, axis=1, keepdims=True)
                k[0, pos, g, :] = (NEEDLE_GAIN * dirs).astype(np.float32)
            kc[b] = bf16_round_bits(k[0])
            vc[b] = bf16_round_bits(v[0])
    return DecodeInputs(name=name, seed=seed, q=bf16_round_bits(kq), k_cache=kc, v_cache=vc,
                        cache_len=np.full((B,), L, dtype=np.int32), block_k=cfg["block_k"],
                        top_k=top_k or cfg["top_k"], sink=cfg["sink"], local=cfg["local"])
