"""Benchmark: one step = the whole sparse-prefill hot path (estimation pass + block-sparse
attention) of one attention layer on seeded synthetic inputs already resident in HBM.

Default workload: Llama-3.1-8B-shaped layer at 128K (batch 1, 32 query / 8 KV heads,
head_dim 128, bf16, block 128x64, sink 32, local 256, per-KV-head theta from {2, 3, 4, 6}).
Prints one JSON line.  --workload selects the other configurations for manual runs
(llama8b_32k, stripe_64k, decode_b16_128k).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_INT8_TOPS = 5000.0       # MI355X dense int8 MFMA
PEAK_FP4_TFLOPS = 10100.0     # MI355X dense fp4 MFMA

PREFILL = ("llama8b_128k", "llama8b_32k", "stripe_64k")
ATTN_SRC = os.path.join(ROOT, "block_sparse_attention_estimate_amd", "csrc", "attn_kernels.hip")
DEC_SRC = os.path.join(ROOT, "block_sparse_attention_estimate_amd", "csrc", "decode_kernels.hip")
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 1 << 30          # plain device copy used to calibrate the byte counters


def source_hash(path):
    import hashlib
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def traffic_from_profile(name, src, key="hbm_bytes_per_launch"):
    """A figure recorded in profiles/<name>.txt (HBM bytes per launch by default), or None
    when missing or taken on a different kernel source."""
    path = os.path.join(PROFILES, name + ".txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != source_hash(src):
        return None
    try:
        return float(kv[key])
    except (KeyError, ValueError):
        return None


def summarize_pmc(fetch_dir, write_dir, kernel, workload, src, command):
    """Text summary of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE in KiB per
    dispatch) for `kernel`, scaled by the same counters on a plain copy of COPY_BYTES."""
    import csv
    import glob

    def per_dispatch(d, counter):
        vals, copy = [], []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                if kernel in r["Kernel_Name"]:
                    vals.append(float(r["Counter_Value"]))
                elif "copyBuffer" in r["Kernel_Name"]:
                    copy.append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
        # the calibration copy is the run's last copy dispatch (after the timed steps)
        return (sum(vals) / len(vals) if vals else float("nan"),
                max(copy)[1] if copy else float("nan"), len(vals))

    f_k, f_c, n_f = per_dispatch(fetch_dir, "FETCH_SIZE")
    w_k, w_c, n_w = per_dispatch(write_dir, "WRITE_SIZE")
    f_scale = COPY_BYTES / (f_c * 1024.0)
    w_scale = COPY_BYTES / (w_c * 1024.0)
    total = f_k * 1024.0 * f_scale + w_k * 1024.0 * w_scale
    lines = [f"# HBM traffic of {kernel} on {workload}",
             f"command: {command}",
             f"kernel_source_sha256_16: {source_hash(src)}",
             f"dispatches: fetch {n_f}, write {n_w}",
             f"fetch_kib_per_dispatch: {f_k:.1f}",
             f"write_kib_per_dispatch: {w_k:.1f}",
             f"copy_fetch_kib ({COPY_BYTES} B copy): {f_c:.1f}",
             f"copy_write_kib ({COPY_BYTES} B copy): {w_c:.1f}",
             f"fetch_scale: {f_scale:.4f}",
             f"write_scale: {w_scale:.4f}",
             f"hbm_bytes_per_launch: {total:.0f}"]
    return "\n".join(lines)


def _pmc_values(d, counter, kernel):
    """Per-dispatch values of `counter` for dispatches whose name contains `kernel`, from the
    counter_collection CSVs of a rocprofv3 --pmc run."""
    import csv
    import glob
    vals = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and kernel in r["Kernel_Name"]:
                vals.append(float(r["Counter_Value"]))
    return vals


def _last_copy(d, counter):
    """`counter` of the run's last copy dispatch (the calibration copy after the timed steps)."""
    import csv
    import glob
    copy = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and "copyBuffer" in r["Kernel_Name"]:
                copy.append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    return max(copy)[1] if copy else float("nan")


def summarize_mfma(util_dir, raw_dir, kernel, workload, src, command):
    """MFMA counters of `kernel`: the derived MfmaUtil (MFMA-busy cycles summed over SIMDs over
    GPU-active cycles times the SIMD count) from one pass, and the bf16 / int8 MFMA operation
    counts (units of 512 flops) and busy cycles from another."""
    util = _pmc_values(util_dir, "MfmaUtil", kernel)
    mops = _pmc_values(raw_dir, "SQ_INSTS_VALU_MFMA_MOPS_BF16", kernel)
    mops8 = _pmc_values(raw_dir, "SQ_INSTS_VALU_MFMA_MOPS_I8", kernel)
    busy = _pmc_values(raw_dir, "SQ_VALU_MFMA_BUSY_CYCLES", kernel)
    avg = lambda v: sum(v) / len(v) if v else float("nan")
    lines = [f"# MFMA counters of {kernel} on {workload}",
             f"command: {command}",
             f"kernel_source_sha256_16: {source_hash(src)}",
             f"dispatches: util {len(util)}, raw {len(mops)}",
             f"mfma_util_percent: {avg(util):.2f}",
             f"mfma_bf16_flops_per_dispatch: {avg(mops) * 512:.4e}",
             f"mfma_i8_ops_per_dispatch: {avg(mops8) * 512:.4e}",
             f"mfma_busy_cycles_sum_over_simds: {avg(busy):.4e}"]
    return "\n".join(lines)


def summarize_kernels(fetch_dir, write_dir, stats_csv, kernels, workload, command):
    """Per-kernel HBM bytes (FETCH_SIZE and WRITE_SIZE per dispatch, scaled by the same counters
    on the calibration copy) over the kernel's average duration from a kernel-trace run."""
    import csv
    dur = {}
    for r in csv.DictReader(open(stats_csv)):
        dur[r["Name"]] = float(r["AverageNs"])
    fc = _last_copy(fetch_dir, "FETCH_SIZE")
    wc = _last_copy(write_dir, "WRITE_SIZE")
    fs, ws = COPY_BYTES / (fc * 1024.0), COPY_BYTES / (wc * 1024.0)
    lines = [f"# HBM bytes and achieved GB/s per kernel on {workload}",
             f"command: {command}",
             f"fetch_scale: {fs:.4f}  write_scale: {ws:.4f}  (1 GiB copy calibration)",
             f"{'kernel':44s} {'fetch_MB':>10s} {'write_MB':>10s} {'avg_us':>10s} {'GB/s':>8s}"]
    for k in kernels:
        f = _pmc_values(fetch_dir, "FETCH_SIZE", k)
        w = _pmc_values(write_dir, "WRITE_SIZE", k)
        if not f or not w:
            continue
        fb = sum(f) / len(f) * 1024.0 * fs
        wb = sum(w) / len(w) * 1024.0 * ws
        names = [n for n in dur if k in n]
        us = dur[names[0]] / 1e3 if names else float("nan")
        lines.append(f"{k:44s} {fb / 1e6:10.1f} {wb / 1e6:10.1f} {us:10.1f} "
                     f"{(fb + wb) / (us * 1e3):8.0f}")
    return "\n".join(lines)


def summarize_stats(stats_csv, title, command):
    """Text summary of a rocprofv3 --kernel-trace --stats run: calls, average duration, total
    and share per kernel (longest total first), with the hashes of the kernel sources."""
    import csv
    rows = sorted(csv.DictReader(open(stats_csv)), key=lambda r: -float(r["TotalDurationNs"]))
    srcs = {n: source_hash(os.path.join(ROOT, "block_sparse_attention_estimate_amd", "csrc", n + ".hip"))
            for n in ("attn_kernels", "est_kernels", "anchor_kernels", "decode_kernels")}
    lines = [f"# Kernel trace summary, {title}",
             f"command: {command}",
             "kernel_sources_sha256_16: " + ", ".join(f"{k} {v}" for k, v in srcs.items()),
             f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'total_ms':>10s} {'pct':>6s}"]
    for r in rows:
        lines.append(f"{r['Name'][:60]:60s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.1f} "
                     f"{float(r['TotalDurationNs']) / 1e6:10.2f} {float(r['Percentage']):6.2f}")
    return "\n".join(lines)


def copy_calibration(dev):
    import torch
    n = COPY_BYTES // 2
    src = torch.ones(n, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


FLUSH_BYTES = 512 << 20       # touched between timed repetitions (larger than the 256 MB MALL)


class CacheFlush:
    """Evicts the inputs from the caches between timed repetitions by touching FLUSH_BYTES of
    another buffer, outside the timed events.  "read" (default) sums the buffer: the caches end
    up full of clean lines, so the next repetition pays no write-back.  "write" fills it: up to
    the memory-side cache's 256 MB of dirty lines are then written back to HBM while the next
    repetition runs, which slows short steps (decode) by the time of that write-back.  "none"
    leaves the caches warm (the two input copies still alternate)."""

    def __init__(self, mode, dev):
        import torch
        self.mode = mode
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev) \
            if mode != "none" else None
        self.sink = torch.zeros((), dtype=torch.float32, device=dev)

    def __call__(self, i):
        import torch
        if self.mode == "read":
            torch.sum(self.buf, dim=0, out=self.sink)
        elif self.mode == "write":
            self.buf.fill_(float(i))

    def describe(self):
        return {"read": f"{FLUSH_BYTES} B read (sum) between reps",
                "write": f"{FLUSH_BYTES} B written (fill) between reps",
                "none": "none (warm caches)"}[self.mode]


class SclkSampler:
    """Samples the GPU shader clock (the active level of the sysfs pp_dpm_sclk table) from a
    thread while the timed repetitions run.  Reports the distinct levels seen (MHz) or None
    when the table is not readable."""

    def __init__(self, period_s=0.005):
        import glob
        import threading
        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thr = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        for pth in self.paths:
            try:
                for line in open(pth):
                    if line.rstrip().endswith("*"):
                        return int(line.split(":")[1].strip().lower().split("mhz")[0])
            except (OSError, ValueError, IndexError):
                continue
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.paths:
            self._thr.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.paths:
            self._thr.join()

    def summary(self):
        if not self.samples:
            return None
        v = np.asarray(self.samples, dtype=np.float64)
        return {"median_mhz": float(np.median(v)), "min_mhz": float(v.min()),
                "max_mhz": float(v.max()), "samples": int(v.size),
                "source": "sysfs pp_dpm_sclk active level, sampled every 5 ms during the timed reps"}


def pct(v):
    """median, p10, p90 of a list of times"""
    a = np.asarray(v, dtype=np.float64)
    return float(np.median(a)), float(np.percentile(a, 10)), float(np.percentile(a, 90))


def useful_pairs_block(counts, idx, stride, N, block_q, block_k):
    """Causal (row, key) pairs inside the kept tiles: sum over kept (b, g, i, J) of the pairs
    (r, j) with r in query block i, j in key block J, j <= r and j < N."""
    c = counts.reshape(-1).astype(np.int64)
    ix = idx.reshape(c.size, stride).astype(np.int64)
    nqb = counts.shape[-1]
    iq = np.tile(np.arange(nqb, dtype=np.int64), c.size // nqb)
    valid = np.arange(stride)[None, :] < c[:, None]
    r0 = (iq * block_q)[:, None]
    r1 = np.minimum(N, (iq + 1) * block_q)[:, None]
    k0 = ix * block_k
    k1 = np.minimum(N, k0 + block_k)

    def tri(x):   # 1 + 2 + ... + x
        return x * (x + 1) // 2
    # rows in [max(r0, k0), min(r1, k1)) see r - k0 + 1 keys of the tile; rows from
    # max(r0, k1) on see all k1 - k0
    lo, hi = np.maximum(r0, k0), np.minimum(r1, k1)
    pairs = np.where(hi > lo, tri(hi - k0) - tri(lo - k0), 0)
    pairs = pairs + np.maximum(r1 - np.maximum(r0, k1), 0) * (k1 - k0)
    return int((pairs * valid).sum())


def cpu_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count()
    return model, affinity


def to_dev(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def cpu_baseline_prefill(x, dense_flops, n_est_rows=None, n_attn_rows=512, seed=1):
    """The oracle (numpy fp64) on the same workload: the estimate over every row (b, g, i)
    (n_est_rows=None) or a random sample of them, timed, and the attention over a random
    sample of query blocks (b, h, i) under the oracle's own lists, timed and scaled by total
    rows / sampled rows to the layer (extrapolated)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = max([int(p.get("num_threads", 1)) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = None
    model, affinity = cpu_info()
    B, N, Hq, D = x.q.shape
    Hkv = x.k.shape[2]
    G = Hq // Hkv
    nqb = -(-N // x.block_q)
    rng = np.random.default_rng(seed)
    kw = dict(block_q=x.block_q, block_k=x.block_k, sink=x.sink, local=x.local,
              granularity=x.granularity)
    all_rows = [(b, g, i) for b in range(B) for g in range(Hkv) for i in range(nqb)]
    if n_est_rows is None or n_est_rows >= len(all_rows):
        rows = all_rows
    else:
        pick = rng.choice(len(all_rows), size=n_est_rows, replace=False)
        rows = sorted(all_rows[j] for j in pick)        # grouped by KV head: tiles quantised once
    t0 = time.perf_counter()
    ref = oracle.estimate_rows(x.q, x.k, x.theta, rows=rows, keep_margins=False, **kw)
    t_est = time.perf_counter() - t0
    # attention sample: random (b, g, i) rows of the estimate, a random head of the group each
    arows = []
    for j in rng.choice(len(rows), size=min(n_attn_rows, len(rows)), replace=False):
        b, g, i = rows[j]
        arows.append((b, g * G + int(rng.integers(0, G)), i))
    # grouped by (b, KV head): the oracle converts one group's keys and values at a time
    arows.sort(key=lambda r: (r[0], r[1] // G, r[1], r[2]))
    lists = {key: r["kept"] for key, r in ref.items()}
    t0 = time.perf_counter()
    oracle.attention_rows(x.q, x.k, x.v, lists, rows=arows, block_q=x.block_q,
                          block_k=x.block_k, granularity=x.granularity)
    t_att = time.perf_counter() - t0
    est_layer = t_est * (B * Hkv * nqb) / len(rows)
    att_layer = t_att * (B * Hq * nqb) / len(arows)
    full = est_layer + att_layer
    est_kind = "measured over every row" if len(rows) == len(all_rows) else \
        f"extrapolated from {len(rows)} random rows"
    return {"value": dense_flops / full / 1e12, "unit": "TFLOP/s (dense-equivalent)",
            "cores": blas, "kind": "oracle",
            "sample": f"estimate: {len(rows)} of {len(all_rows)} rows (b,g,i) in {t_est:.1f}s "
                      f"({est_kind}); attention: {len(arows)} random query blocks (b,h,i) in "
                      f"{t_att:.1f}s, extrapolated by rows to the layer ({att_layer:.0f}s); "
                      f"layer {full:.0f}s",
            "cpu_model": model, "affinity_cores": affinity, "blas_threads": blas,
            "estimate_s": round(est_layer, 2), "estimate_measured": len(rows) == len(all_rows),
            "attention_s_extrapolated": round(att_layer, 1)}


def cpu_one_thread(seed=1):
    """The oracle with its BLAS limited to one thread on the two smaller prefill
    configurations: the 4K tiny layer in full (estimate and attention, measured) and the 32K
    layer on 256 random estimate rows and 128 random attention query blocks (scaled by rows to
    the layer).  Returns seconds per layer for each leg."""
    import oracle
    import synth
    from threadpoolctl import threadpool_limits
    out = {"blas_threads": 1}
    with threadpool_limits(1):
        x = synth.make_prefill("tiny_4k")
        kw = dict(block_q=x.block_q, block_k=x.block_k, sink=x.sink, local=x.local)
        t0 = time.perf_counter()
        ref = oracle.estimate_all(x.q, x.k, x.theta, **kw)
        t_est = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.attention_all(x.q, x.k, x.v, {k: r["kept"] for k, r in ref.items()},
                             block_q=x.block_q, block_k=x.block_k)
        t_att = time.perf_counter() - t0
        out["tiny_4k"] = {"estimate_s": round(t_est, 3), "attention_s": round(t_att, 3),
                          "kind": "measured over the whole layer"}
        x = synth.make_prefill("llama8b_32k")
        B, N, Hq, D = x.q.shape
        Hkv = x.k.shape[2]
        G = Hq // Hkv
        nqb = -(-N // x.block_q)
        kw = dict(block_q=x.block_q, block_k=x.block_k, sink=x.sink, local=x.local)
        rng = np.random.default_rng(seed)
        all_rows = [(b, g, i) for b in range(B) for g in range(Hkv) for i in range(nqb)]
        rows = sorted(all_rows[j] for j in rng.choice(len(all_rows), size=256, replace=False))
        t0 = time.perf_counter()
        ref = oracle.estimate_rows(x.q, x.k, x.theta, rows=rows, keep_margins=False, **kw)
        t_est = time.perf_counter() - t0
        arows = []
        for j in rng.choice(len(rows), size=128, replace=False):
            b, g, i = rows[j]
            arows.append((b, g * G + int(rng.integers(0, G)), i))
        arows.sort(key=lambda r: (r[0], r[1] // G, r[1], r[2]))
        t0 = time.perf_counter()
        oracle.attention_rows(x.q, x.k, x.v, {k: r["kept"] for k, r in ref.items()}, rows=arows,
                              block_q=x.block_q, block_k=x.block_k)
        t_att = time.perf_counter() - t0
        out["llama8b_32k"] = {"estimate_s": round(t_est * len(all_rows) / len(rows), 2),
                              "attention_s": round(t_att * B * Hq * nqb / len(arows), 2),
                              "kind": "256 estimate rows and 128 attention query blocks, "
                                      "scaled by rows to the layer"}
    return out


def bench_prefill(args, dev):
    import torch
    import block_sparse_attention_estimate_amd as sa
    import synth
    log(f"generating {args.workload}")
    x = synth.make_prefill(args.workload, seed=args.seed)
    B, N, Hq, D = x.q.shape
    Hkv = x.k.shape[2]
    G = Hq // Hkv
    q, k, v = to_dev(x.q, dev), to_dev(x.k, dev), to_dev(x.v, dev)
    kw = dict(block_q=x.block_q, block_k=x.block_k, sink=x.sink, local=x.local)
    if args.theta is not None:
        x.theta = np.full(Hq, args.theta, np.float32)
    est = args.estimator
    stride = None
    if x.granularity == "stripe":
        stride = args.stripe_capacity
    reuse = args.anchor_reuse
    if reuse and est != "pooled":
        raise SystemExit("--anchor-reuse needs the pooled estimator")
    lists = sa.alloc_lists(q, k, block_q=x.block_q, block_k=x.block_k,
                           granularity=x.granularity, stride=stride)
    op = sa.SA_OP_ESTIMATE_STATE if reuse else sa.SA_OP_ESTIMATE
    ws = torch.empty(sa.workspace_size(op, q=q, k=k, granularity=x.granularity,
                                       estimator=est, **kw), dtype=torch.uint8, device=dev)
    state = sa.alloc_anchor_state(q) if reuse else None
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    # two copies of the inputs, used alternately, and a 512 MB write between repetitions, so
    # that no repetition finds its inputs in the caches (the MALL holds 256 MB)
    copies = [(q, k, v), tuple(t.clone() for t in (q, k, v))]
    flush = CacheFlush(args.flush, dev)

    def step(i, ev=None):
        qq, kk, vv = copies[i % 2]
        if ev is not None:
            ev[0].record(stream)
        if reuse:
            sa.estimate_mask_anchor_state(qq, kk, vv, x.theta, granularity=x.granularity,
                                          step=args.step, workspace=ws, out=lists, state=state,
                                          **kw)
        else:
            sa.estimate_mask(qq, kk, x.theta, granularity=x.granularity, estimator=est,
                             step=args.step, workspace=ws, out=lists, **kw)
        if ev is not None:
            ev[1].record(stream)
        if reuse:
            sa.sparse_prefill_resume(qq, kk, vv, lists, state, out=o, lse=False, **kw)
        else:
            sa.sparse_prefill(qq, kk, vv, lists, out=o, lse=False, **kw)
        if ev is not None:
            ev[2].record(stream)

    log("warmup")
    for i in range(args.warmup):
        step(i)
        flush(i)
    torch.cuda.synchronize()
    if x.granularity == "stripe" and lists.overflowed():
        raise SystemExit("stripe list capacity exceeded; raise --stripe-capacity")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    with SclkSampler() as sclk:
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i, evs[i])
            flush(i)                            # outside the timed events
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    est_ms = [e[0].elapsed_time(e[1]) for e in evs]
    att_ms = [e[1].elapsed_time(e[2]) for e in evs]
    step_ms = [e[0].elapsed_time(e[2]) for e in evs]
    ms_step, p10_step, p90_step = pct(step_ms)
    counts = lists.counts.cpu().numpy().astype(np.int64)
    nqb = counts.shape[2]
    ends = np.minimum(N, (np.arange(nqb) + 1) * x.block_q) - 1
    if x.granularity == "block":
        cands = (ends // x.block_k + 1).astype(np.int64)
        kept_units = int(counts.sum()) * G                       # kept (head, 128x64 tile)
        flops_per_unit = 4.0 * x.block_q * x.block_k * D
        density = float(counts.sum() / (cands.sum() * B * Hkv))
    else:
        cands = (ends + 1).astype(np.int64)
        kept_units = int(counts.sum()) * G                       # kept (head, column)
        flops_per_unit = 4.0 * x.block_q * D
        density = float(counts.sum() / (cands.sum() * B * Hkv))
    kept_flops = kept_units * flops_per_unit
    unit_name = f"(head, {x.block_q}x{x.block_k} tile)" if x.granularity == "block" else \
        f"(head, {x.block_q}-row column)"
    units_desc = f"{kept_units} kept {unit_name} x {flops_per_unit / 1e6:.3f} MFLOP"
    if reuse:
        # the resuming pass visits, per 64-row work item, the listed tiles that start before
        # the item's last row's local window and do not lie inside the sink tokens (block
        # lists), or the listed columns in [sink, last row - local] (column lists)
        idx = lists.idx.cpu().numpy().reshape(-1, lists.stride).astype(np.int64)
        cnt = counts.reshape(-1)
        valid = np.arange(lists.stride)[None, :] < cnt[:, None]
        iq = np.tile(np.arange(nqb), B * Hkv)
        visited = 0
        for tsub in range(x.block_q // 64):
            r0 = iq * x.block_q + tsub * 64
            ok_row = r0 < N
            cut = np.minimum(r0 + 63, N - 1) - x.local + 1
            if x.granularity == "block":
                vis = valid & (idx * 64 < cut[:, None]) & (idx * 64 + 63 >= x.sink)
            else:
                vis = valid & (idx < cut[:, None]) & (idx >= x.sink)
            visited += int((vis & ok_row[:, None]).sum())
        kept_units = visited * G
        if x.granularity == "block":
            flops_per_unit = 4.0 * 64 * x.block_k * D             # (head, 64-row, 64-key tile)
            units_desc = (f"{kept_units} visited (head, 64x{x.block_k} tile) x "
                          f"{flops_per_unit / 1e6:.3f} MFLOP (the anchor state covers the rest)")
        else:
            flops_per_unit = 4.0 * 64 * D                         # (head, 64-row item, column)
            units_desc = (f"{kept_units} visited (head, 64-row item, column) x "
                          f"{flops_per_unit / 1e3:.1f} KFLOP (the anchor state covers the rest)")
        kept_flops = kept_units * flops_per_unit
    dense_flops = 2.0 * N * N * D * Hq * B
    att_avg, att_p10, att_p90 = pct(att_ms)
    est_avg, est_p10, est_p90 = pct(est_ms)
    achieved = kept_flops / (att_avg * 1e-3) / 1e12
    per_group = (counts.sum(axis=(0, 2)) / (cands.sum() * B)).round(4).tolist()
    useful = None
    if x.granularity == "block" and not reuse:
        # causal (row, key) pairs inside the kept tiles, 4 d flops each per query head
        pairs = useful_pairs_block(counts, lists.idx.cpu().numpy(), lists.stride, N, x.block_q,
                                   x.block_k)
        useful = 4.0 * D * pairs * G
    theta_g = [round(float(t), 3) for t in x.theta.reshape(Hkv, G)[:, 0]] \
        if np.all(x.theta.reshape(Hkv, G) == x.theta.reshape(Hkv, G)[:, :1]) else \
        [round(float(t), 3) for t in x.theta]
    theta_desc = (f"theta per KV head {theta_g}" if len(theta_g) == Hkv else
                  f"theta per query head {theta_g}")
    # the attention kernel the library launches for these lists
    kernel = "attn_block"
    out = {
        "metric": "ms/layer & dense-equiv TFLOP/s (fraction of MFMA peak) for sparse prefill @128K",
        "value": round(dense_flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s (dense-equivalent)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.workload}: batch {B}, {Hq}/{Hkv} heads, d {D}, "
                               f"seq {N}, block {x.block_q}x{x.block_k}, sink {x.sink}, "
                               f"local {x.local}, {x.granularity}, {est} estimator, " + theta_desc +
                               (f", step {args.step}" if args.step > 1 else "") +
                               (", anchor-state reuse" if reuse else ""),
                   "global_batch": B, "seq_len": N, "parallelism": "none (1 GPU)"},
        "ms_per_layer": round(ms_step, 3),
        "timing": {"reps": args.steps, "statistic": "median of per-repetition HIP event times "
                                                    "on the library's stream",
                   "step_ms_median_p10_p90": [round(ms_step, 3), round(p10_step, 3), round(p90_step, 3)],
                   "estimate_ms_median_p10_p90": [round(est_avg, 3), round(est_p10, 3), round(est_p90, 3)],
                   "attention_ms_median_p10_p90": [round(att_avg, 3), round(att_p10, 3), round(att_p90, 3)],
                   "step_ms_mean": round(float(np.mean(step_ms)), 3),
                   "wall_ms_per_rep_incl_flush": round(wall * 1e3 / args.steps, 3),
                   "input_copies": 2, "flush_between_reps": flush.describe(),
                   "sclk": sclk.summary()},
        "estimate_ms": round(est_avg, 3), "attention_ms": round(att_avg, 3),
        "estimate_over_attention": round(est_avg / att_avg, 4),
        "kept_density": round(density, 5), "kept_density_per_kv_head": per_group,
        "kept_tile_tflops": round(achieved, 2),
        "kept_tile_frac_of_bf16_peak": round(achieved / PEAK_BF16_TFLOPS, 4),
        "useful_pair_tflops": None if useful is None else round(useful / (att_avg * 1e-3) / 1e12, 2),
        "useful_pair_flops": useful,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None if reuse else
                                traffic_from_profile(f"{kernel}_{args.workload}_traffic", ATTN_SRC),
                     "mfma_util_percent_counter": None if reuse else
                                traffic_from_profile(f"{kernel}_{args.workload}_mfma", ATTN_SRC,
                                                     "mfma_util_percent"),
                     "kernel": f"{kernel} (sa_sparse_prefill_resume)" if reuse
                               else f"{kernel} (sa_sparse_prefill)",
                     "units": units_desc},
    }
    if est != "pooled":
        # the element-wise estimate: 2 d ops per causal (row, key) pair and query head, on
        # int8 or block-scaled fp4 MFMA
        pairs = float(N) * (N + 1) / 2
        est_ops = 2.0 * D * pairs * Hq * B
        peak, kind = (PEAK_INT8_TOPS, "int8") if est == "relative" else (PEAK_FP4_TFLOPS, "fp4")
        out[f"estimate_{kind}_tops"] = round(est_ops / (est_avg * 1e-3) / 1e12, 1)
        out[f"estimate_frac_of_{kind}_peak"] = round(est_ops / (est_avg * 1e-3) / 1e12 / peak, 4)
    if args.cpu_baseline:
        log("cpu baseline (oracle sample)")
        out["cpu_baseline"] = cpu_baseline_prefill(x, dense_flops)
        log("oracle with one BLAS thread (tiny 4K, 32K sample)")
        out["cpu_baseline"]["one_thread"] = cpu_one_thread()
    return out


def _decode_params(x, kw):
    from block_sparse_attention_estimate_amd import _lib
    p = _lib.SaDecodeParams()
    p.block_k, p.top_k_blocks, p.sink_tokens, p.local_tokens = (kw["block_k"], kw["top_k"],
                                                                 kw["sink"], kw["local"])
    p.n_splits, p.softmax_scale, p.top_p = kw["n_splits"], 0.0, float(kw["top_p"] or 0.0)
    return p


def bench_decode(args, dev):
    import torch
    import block_sparse_attention_estimate_amd as sa
    import synth
    log("generating decode workload")
    x = synth.make_decode(args.workload, seed=args.seed)
    B, Hq, D = x.q.shape
    L, Hkv = x.k_cache.shape[1], x.k_cache.shape[2]
    q, kc, vc = to_dev(x.q, dev), to_dev(x.k_cache, dev), to_dev(x.v_cache, dev)
    cl = torch.from_numpy(x.cache_len).to(dev)
    kbar = sa.build_block_summary(kc, cl, block_k=x.block_k)
    if args.summary == "q4":
        kbar = sa.quantize_block_summary(kbar, block_k=x.block_k)
    elif args.summary == "fp4":
        kbar = sa.quantize_block_summary_fp4(kbar, block_k=x.block_k)
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    top_k = args.top_k or x.top_k
    kw = dict(block_k=x.block_k, top_k=top_k, sink=x.sink, local=x.local, top_p=args.top_p,
              n_splits=args.n_splits)
    o, lse, sel = sa.sparse_decode(q, kc, vc, kbar, cl, out=o, **kw)
    n_sel = int((sel >= 0).sum().item())                 # blocks selected over all (b, g)
    # two copies of the caches and summaries, used alternately, and a 512 MB write between
    # repetitions: the selected K/V (256 MiB) and the summaries would otherwise sit in the MALL
    kc2, vc2 = kc.clone(), vc.clone()
    kbar2 = tuple(t.clone() for t in kbar) if isinstance(kbar, tuple) else kbar.clone()
    copies = [(q, kc, vc, kbar), (q.clone(), kc2, vc2, kbar2)]
    flush = CacheFlush(args.flush, dev)
    ws = torch.empty(sa.workspace_size(sa.SA_OP_DECODE, shape=sa._decode_shape(q, kc, vc, o),
                                       decode_params=_decode_params(x, kw)),
                     dtype=torch.uint8, device=dev)
    for i in range(args.warmup):
        qq, kk, vv, kb = copies[i % 2]
        sa.sparse_decode(qq, kk, vv, kb, cl, out=o, workspace=ws, return_selected=False, **kw)
        flush(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    with SclkSampler() as sclk:
        for i in range(args.steps):
            qq, kk, vv, kb = copies[i % 2]
            evs[i][0].record(stream)
            sa.sparse_decode(qq, kk, vv, kb, cl, out=o, workspace=ws, return_selected=False, **kw)
            evs[i][1].record(stream)
            flush(i)
        torch.cuda.synchronize()
    rep_us = [e0.elapsed_time(e1) * 1e3 for e0, e1 in evs]
    us, us_p10, us_p90 = pct(rep_us)
    nkb = -(-L // x.block_k)
    sel_bytes = n_sel * x.block_k * D * 2 * 2
    per_row = {"bf16": D * 2, "q4": D // 2 + D // 32 * 2, "fp4": D // 2 + D // 32}[args.summary]
    sum_bytes = B * Hkv * nkb * per_row
    gbs = (sel_bytes + sum_bytes) / (us * 1e-6) / 1e9
    return {"metric": "sparse decode step time and achieved HBM GB/s",
            "value": round(gbs, 1), "unit": "GB/s (algorithmic)", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(us / 1e3, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": f"{args.workload}: batch {B}, {Hq}/{Hkv} heads, d {D}, "
                                   f"cache {L}, " + (f"top-{top_k} blocks of {x.block_k}, "
                                   if args.top_p == 0 else f"top-p {args.top_p} budget (at most "
                                   f"{top_k} blocks of {x.block_k}), ") +
                                   f"{args.summary} block summaries",
                       "global_batch": B, "seq_len": L, "parallelism": "none (1 GPU)"},
            "us_per_step": round(us, 2),
            "timing": {"reps": args.steps, "statistic": "median of per-repetition HIP event times "
                                                        "on the library's stream",
                       "us_median_p10_p90": [round(us, 2), round(us_p10, 2), round(us_p90, 2)],
                       "us_mean": round(float(np.mean(rep_us)), 2),
                       "input_copies": 2, "flush_between_reps": flush.describe(),
                       "sclk": sclk.summary()},
            "mean_blocks_selected": round(n_sel / (B * Hkv), 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": traffic_from_profile(f"dec_splitk_{args.workload}_traffic", DEC_SRC),
                         "kernel": "whole decode step (score, select, split-K, combine: one "
                                   "library call, timed as one)",
                         "units": f"{sel_bytes} B of selected K/V + {sum_bytes} B of block "
                                  f"summaries per step"}}


def bench_calibrate(args, dev):
    """Per-head theta calibration (sa_calibrate_theta) on a prefill workload: wall time of the
    whole loop, rounds, calibrated thetas, halvings and final errors."""
    import math
    import torch
    import block_sparse_attention_estimate_amd as sa
    import synth
    log(f"generating {args.workload}")
    x = synth.make_prefill(args.workload, seed=args.seed)
    B, N, Hq, D = x.q.shape
    q, k, v = to_dev(x.q, dev), to_dev(x.k, dev), to_dev(x.v, dev)
    kw = dict(block_q=x.block_q, block_k=x.block_k, sink=x.sink, local=x.local)
    sa.calibrate_theta(q, k, v, tau0=0.008, err_bound=args.err_bound, max_halvings=0, **kw)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    th, err, hv = sa.calibrate_theta(q, k, v, tau0=0.008, err_bound=args.err_bound,
                                     max_halvings=args.max_halvings, **kw)
    wall = time.perf_counter() - t0
    rounds = int(hv.max()) + 1
    return {"metric": "per-head theta calibration wall time (tau from 0.008 halved until "
                      "Err <= bound)", "value": round(wall * 1e3, 2), "unit": "ms",
            "n_gpus": 1, "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"{args.workload}: batch {B}, {Hq}/{x.k.shape[2]} heads, "
                                   f"d {D}, seq {N}", "err_bound": args.err_bound,
                       "max_halvings": args.max_halvings},
            "rounds": rounds, "ms_per_round": round(wall * 1e3 / (rounds + 1), 2),
            "theta": [round(float(t), 4) for t in th], "halvings": hv.tolist(),
            "err": [round(float(e), 5) for e in err],
            "theta0": round(-math.log(0.008), 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama8b_128k",
                    choices=list(PREFILL) + ["decode_b16_128k"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--stripe-capacity", type=int, default=8192)
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--flush", choices=["read", "write", "none"], default="read",
                    help="how the caches are flushed between timed repetitions")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run one plain 1 GiB device copy (byte-counter scale)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the traffic summary of two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("UTIL_DIR", "RAW_DIR"),
                    help="print the MFMA counter summary of two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-kernels", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "STATS_CSV"),
                    help="print per-kernel HBM bytes and GB/s for --kernels and exit")
    ap.add_argument("--summarize-stats", metavar="STATS_CSV",
                    help="print the kernel table of a rocprofv3 --kernel-trace --stats run and exit")
    ap.add_argument("--title", default="", help="title line of --summarize-stats")
    ap.add_argument("--kernels", default="est_quant_k,est_anchor_pool,est_score_block,est_compact")
    ap.add_argument("--kernel", default="attn_block")
    ap.add_argument("--summary", choices=["bf16", "q4", "fp4"], default="bf16",
                    help="decode: block summaries in bf16, 4-bit codes + bf16 scales (q4) or MXFP4 (fp4)")
    ap.add_argument("--estimator", choices=["pooled", "relative", "relative_mxfp4"],
                    default="pooled",
                    help="prefill: anchor vs pooled query, or the element-wise relative score "
                         "(int8 or MXFP4 operands)")
    ap.add_argument("--anchor-reuse", action="store_true",
                    help="estimate with the anchor state and resume the prefill from it")
    ap.add_argument("--step", type=int, default=1,
                    help="prefill: identify query blocks in groups of STEP (AnchorAttention)")
    ap.add_argument("--theta", type=float, default=None,
                    help="prefill: one theta for every head instead of the workload's")
    ap.add_argument("--top-p", type=float, default=0.0,
                    help="decode: per-(b, KV head) budget from the block-score distribution")
    ap.add_argument("--n-splits", type=int, default=0,
                    help="decode: splits per (b, KV head) (0: the library's choice)")
    ap.add_argument("--top-k", type=int, default=0,
                    help="decode: block cap (default: the workload's K)")
    ap.add_argument("--calibrate", action="store_true",
                    help="time the per-head theta calibration on the prefill workload instead")
    ap.add_argument("--err-bound", type=float, default=0.4)
    ap.add_argument("--max-halvings", type=int, default=24)
    ap.add_argument("--command", default="")
    args = ap.parse_args()
    if args.summarize_pmc:
        src = DEC_SRC if args.kernel.startswith("dec_") else ATTN_SRC
        print(summarize_pmc(*args.summarize_pmc, args.kernel, args.workload, src, args.command))
        return
    if args.summarize_mfma:
        src = DEC_SRC if args.kernel.startswith("dec_") else ATTN_SRC
        print(summarize_mfma(*args.summarize_mfma, args.kernel, args.workload, src, args.command))
        return
    if args.summarize_kernels:
        print(summarize_kernels(*args.summarize_kernels, args.kernels.split(","), args.workload,
                                args.command))
        return
    if args.summarize_stats:
        print(summarize_stats(args.summarize_stats, args.title, args.command))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the workload "
              "would shard by KV head with no exchange); run with --gpus 1", file=sys.stderr)
        raise SystemExit(2)
    import torch
    dev = torch.device("cuda:0")
    import block_sparse_attention_estimate_amd as sa
    sa.load_library()
    if args.calibrate:
        out = bench_calibrate(args, dev)
    elif args.workload in PREFILL:
        out = bench_prefill(args, dev)
    else:
        out = bench_decode(args, dev)
    if args.copy_calibration:
        copy_calibration(dev)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
