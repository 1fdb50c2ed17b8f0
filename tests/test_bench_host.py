"""Host logic of bench.py on the CPU: the one-GPU refusal, the algorithmic bytes the roofline divides
by, the per-workgroup timeline analysis and the rocprofv3 summaries (on synthetic records and CSV
files; nothing here touches a GPU)."""
from __future__ import annotations

import csv
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2 and ("one GPU" in r.stderr or "single MI355X" in r.stderr), r.stderr


def test_required_bytes_by_hand():
    # 128K, Max, SHARED, k 96: 991 candidates; 128 + 96*128 + 4096 = 16512 attended tokens per KV head
    rb = bench.required_bytes(bench.WORKLOADS["128k-max"])
    assert (rb["ncand"], rb["k_eff"], rb["tokens"]) == (991, 96, 16512)
    assert rb["kv"] == 8 * 16512 * 256 * 2 and rb["reps"] == 991 * 8 * 128 * 2
    assert bench.required_per_step("128k-max") == 69_687_296
    # Quest at 1M: two fp16 rep rows per (block, KV head), 32 layers
    rb = bench.required_bytes(bench.WORKLOADS["1m"])
    assert rb["reps"] == 8159 * 8 * 2 * 128 * 2
    assert bench.required_per_step("1m") == 32 * 84_299_776
    # quantized rows: codes plus scales (and the INT4 zero point) per token row of one KV head
    for name, row in (("128k-max-q8", 128 + 8), ("128k-max-q4", 64 + 8), ("128k-max-i8", 128 + 4),
                      ("128k-max-i4", 64 + 4 + 1)):
        assert bench.required_bytes(bench.WORKLOADS[name])["kv"] == 8 * 16512 * row * 2, name
    # the batched workload: a window's mean, at least its first step's decode bytes
    w = bench.WORKLOADS["mixed"]
    lens = bench.mixed_lengths(w)
    assert len(lens) == 16 and all(w["Lmin"] <= L <= w["Lmax"] for L in lens)
    first = sum(sum(bench.required_bytes(w, L)[k] for k in ("q", "reps", "kv", "out")) for L in lens)
    assert first <= bench.required_per_step("mixed") <= first * 1.01


def _records(spec, n_kinds=len(bench.TL_KINDS)):
    rec = np.zeros((n_kinds, bench.TL_MAX_WG, bench.TL_SLOTS))
    for kind, idx, slots in spec:
        for slot, t in slots.items():
            rec[kind, idx, slot] = t
    return rec


def test_timeline_analysis():
    base = 1e6  # ticks of the 100 MHz clock
    spec = [
        (0, 0, {0: base, 1: base + 300, 2: base + 450}),               # scoring workgroups
        (0, 1, {0: base + 10, 1: base + 400, 2: base + 500, 3: base + 700}),  # the last one selects
        (1, 0, {0: base + 50, 1: base + 250, 2: base + 600}),          # an Initial/Local tile
        (3, 0, {0: base + 900, 1: base + 1300, 2: base + 1500}),       # attention
        (3, 1, {0: base - 5000, 2: base - 4000}),                      # an earlier step's record
        (4, 0, {0: base + 1650, 2: base + 1900}),                      # merge
    ]
    v = bench.timeline_replay_stats(_records(spec))
    assert v[(0, "n")] == 2 and v[(3, "n")] == 1  # the stale attention record is dropped
    assert v[(0, 0)] == (0.0, 0.05, 0.1) and v[(0, 3)] == (7.0, 7.0, 7.0) and v[(0, "end")] == 7.0
    assert v[(3, 0)] == (9.0, 9.0, 9.0) and v[(3, "end")] == 15.0
    med = bench.timeline_medians([v, v, v])
    assert med == v
    text = "\n".join(bench.timeline_lines(med))
    assert "| scoring+selection    | start   0.00 | end   7.00 | span   7.00 | gap      - |" in text
    assert "| attention            | start   9.00 | end  15.00 | span   6.00 | gap   2.00 |" in text
    assert "| merge                | start  16.50 | end  19.00 | span   2.50 | gap   1.50 |" in text
    assert "layer: 19.00 us" in text


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=list(rows[0]))
        wr.writeheader()
        wr.writerows(rows)


def test_profile_summaries(tmp_path):
    d = tmp_path / "prof"
    d.mkdir()
    stat = lambda name, calls, avg: {"Name": name, "Calls": calls, "AverageNs": avg, "MinNs": avg, "MaxNs": avg}
    _write_csv(d / "run_kernel_stats.csv", [
        stat("void kvs::score_select_kernel<4, 1, 1, 0, false>(kvs::AttnArgs, ...)", 100, 8000.0),
        stat("void kvs::attn_tiles_kernel<4, false, true, 0>(kvs::AttnArgs)", 100, 12000.0),
        stat("kvs::merge_wave_kernel(kvs::AttnArgs, int)", 100, 4000.0),
        stat("void kvs::build_reps_kernel<1, 0>(void const*, ...)", 3, 45000.0),  # set-up only
        stat("__amd_rocclr_copyBuffer", 1, 1e6),
    ])
    bench.summarize_stats(str(d), "128k-max", None, 480, out_dir=str(tmp_path))
    txt = open(tmp_path / "decode_step_128k-max_kernel_stats.txt").read()
    assert "sum_of_kernel_averages_us_per_layer: 24.00" in txt
    assert "build_reps_kernel *" in txt and "copyBuffer" not in txt
    fd, wd = tmp_path / "fetch", tmp_path / "write"
    fd.mkdir()
    wd.mkdir()
    copy_kib = bench.COPY_BYTES / 1024.0

    def rows(counter, copy_frac, per_kernel):
        out = [{"Counter_Name": counter, "Counter_Value": copy_kib * copy_frac, "Kernel_Name": "__amd_rocclr_copyBuffer"}]
        for name, kib, n in per_kernel:
            out += [{"Counter_Name": counter, "Counter_Value": kib, "Kernel_Name": name}] * n
        return out

    ks = "void kvs::score_select_kernel<4, 1, 1, 0, false>(kvs::AttnArgs)"
    ka = "void kvs::attn_tiles_kernel<4, false, true, 0>(kvs::AttnArgs)"
    kr = "void kvs::build_reps_kernel<1, 0>(void const*)"
    # FETCH_SIZE reads half of the copy's bytes (scale 2), WRITE_SIZE all of them (scale 1)
    _write_csv(fd / "run_counter_collection.csv", rows("FETCH_SIZE", 0.5, [(ks, 1000.0, 10), (ka, 24000.0, 10),
                                                                          (kr, 99999.0, 1)]))
    _write_csv(wd / "run_counter_collection.csv", rows("WRITE_SIZE", 1.0, [(ks, 300.0, 10), (ka, 800.0, 10),
                                                                          (kr, 99999.0, 1)]))
    bench.summarize_pmc(str(fd), str(wd), "128k-max", 32, out_dir=str(tmp_path))
    kv = bench.read_kv_file(str(tmp_path / "decode_step_128k-max_traffic.txt"))
    assert float(kv["fetch_scale"]) == 2.0 and float(kv["write_scale"]) == 1.0
    assert float(kv["fetch_bytes_per_layer"]) == (1000.0 + 24000.0) * 1024 * 2
    assert float(kv["write_bytes_per_layer"]) == (300.0 + 800.0) * 1024
    want = ((1000.0 + 24000.0) * 2048 + (300.0 + 800.0) * 1024) / 69_687_296
    assert abs(float(kv["traffic_over_required"]) - want) < 1e-4
