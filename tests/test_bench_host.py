"""Host-side logic of bench.py (CPU): the counter summaries that feed the roofline's
`traffic` and MFMA figures, the source-hash guard on stored profiles, and the one-GPU exit."""
import csv
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write_counters(d, rows):
    """A rocprofv3 --pmc output folder with one counter_collection CSV of (kernel, counter, value)."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for i, (k, c, v) in enumerate(rows):       # dispatches in the order given
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": k, "Counter_Name": c,
                        "Counter_Value": v})


def _kv(text):
    out = {}
    for line in text.splitlines():
        if ":" in line:
            k, v = line.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def test_summarize_pmc_scales_by_the_copy(tmp_path):
    # FETCH_SIZE reads half the copy's bytes (scale 2), WRITE_SIZE all of them (scale 1); the
    # kernel's two dispatches average to 3000 KiB fetched and 500 KiB written.  The calibration
    # copy is the run's last copy dispatch: earlier copies (input copies, larger or smaller)
    # do not count.
    copy_kib = bench.COPY_BYTES / 1024
    _write_counters(tmp_path / "f", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 3.0),
                                     ("__amd_rocclr_copyBuffer", "FETCH_SIZE", copy_kib * 4),
                                     ("void attn_block<128, 4, false, false>(AttnArgs)", "FETCH_SIZE", 2000),
                                     ("void attn_block<128, 4, false, false>(AttnArgs)", "FETCH_SIZE", 4000),
                                     ("est_compact(EstArgs)", "FETCH_SIZE", 99999),
                                     ("__amd_rocclr_copyBuffer", "FETCH_SIZE", copy_kib / 2)])
    _write_counters(tmp_path / "w", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", copy_kib * 8),
                                     ("void attn_block<128, 4, false, false>(AttnArgs)", "WRITE_SIZE", 500),
                                     ("void attn_block<128, 4, false, false>(AttnArgs)", "WRITE_SIZE", 500),
                                     ("__amd_rocclr_copyBuffer", "WRITE_SIZE", copy_kib)])
    text = bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), "attn_block", "w",
                               bench.ATTN_SRC, "cmd")
    kv = _kv(text)
    assert kv["dispatches"] == "fetch 2, write 2"
    assert float(kv["fetch_scale"]) == pytest.approx(2.0)
    assert float(kv["write_scale"]) == pytest.approx(1.0)
    assert float(kv["hbm_bytes_per_launch"]) == pytest.approx(3000 * 1024 * 2 + 500 * 1024)
    assert kv["kernel_source_sha256_16"] == bench.source_hash(bench.ATTN_SRC)


def test_traffic_from_profile_needs_the_same_source(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel one\n")
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "p.txt").write_text(f"# x\nkernel_source_sha256_16: {bench.source_hash(str(src))}\n"
                                f"hbm_bytes_per_launch: 12345\nmfma_util_percent: 50.5\n")
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    assert bench.traffic_from_profile("p", str(src)) == 12345.0
    assert bench.traffic_from_profile("p", str(src), key="mfma_util_percent") == 50.5
    assert bench.traffic_from_profile("missing", str(src)) is None
    src.write_text("kernel two\n")          # the kernel changed since the counters were taken
    assert bench.traffic_from_profile("p", str(src)) is None


def test_summarize_mfma(tmp_path):
    k = "void attn_block<128, 4, false, false>(AttnArgs)"
    _write_counters(tmp_path / "u", [(k, "MfmaUtil", 50.0), (k, "MfmaUtil", 60.0)])
    _write_counters(tmp_path / "r", [(k, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1000.0),
                                     (k, "SQ_INSTS_VALU_MFMA_MOPS_I8", 0.0),
                                     (k, "SQ_VALU_MFMA_BUSY_CYCLES", 7.0)])
    kv = _kv(bench.summarize_mfma(str(tmp_path / "u"), str(tmp_path / "r"), "attn_block", "w",
                                  bench.ATTN_SRC, "cmd"))
    assert float(kv["mfma_util_percent"]) == pytest.approx(55.0)
    assert float(kv["mfma_bf16_flops_per_dispatch"]) == pytest.approx(512000.0)
    assert float(kv["mfma_busy_cycles_sum_over_simds"]) == pytest.approx(7.0)


def test_stored_profiles_name_their_command_and_source():
    # every committed summary says how it was made; the ones bench.py reads carry a source hash
    for name in os.listdir(os.path.join(ROOT, "profiles")):
        text = open(os.path.join(ROOT, "profiles", name)).read()
        assert "command:" in text.splitlines()[1], name
        if name.startswith(("attn_block_", "dec_splitk_")):     # the files bench.py reads
            assert "kernel_source_sha256_16:" in text, name


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_useful_pairs_block_brute_force():
    """bench.useful_pairs_block counts the causal (row, key) pairs inside kept tiles: checked
    against a loop over rows and keys on random lists, ragged ends and 32-key blocks."""
    import numpy as np
    rng = np.random.default_rng(0)
    for N, bq, bk in [(1000, 128, 64), (777, 64, 32), (4096, 128, 64), (130, 64, 64), (1, 64, 64)]:
        nqb, nkb = -(-N // bq), -(-N // bk)
        counts = np.zeros((2, 2, nqb), np.int32)
        idx = np.zeros((2, 2, nqb, nkb), np.int32)
        want = 0
        for b in range(2):
            for g in range(2):
                for i in range(nqb):
                    r0, r1 = i * bq, min(N, (i + 1) * bq)
                    cand = np.arange((r1 - 1) // bk + 1)
                    kept = np.sort(rng.choice(cand, size=rng.integers(0, len(cand) + 1), replace=False))
                    counts[b, g, i] = len(kept)
                    idx[b, g, i, :len(kept)] = kept
                    for J in kept:
                        for r in range(r0, r1):
                            for j in range(J * bk, min(N, J * bk + bk)):
                                want += j <= r
        assert bench.useful_pairs_block(counts, idx, nkb, N, bq, bk) == want
