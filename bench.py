#!/usr/bin/env python3
"""Sparse decode benchmark on one MI355X: queries/s and HBM roofline fraction at 128K and 1M tokens.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu] [--no-reuse]
    python bench.py --summarize-stats DIR --workload NAME      (rocprofv3 --stats CSVs -> profiles/)
    python bench.py --summarize-pmc FETCH_DIR WRITE_DIR --workload NAME   (counters -> profiles/)

A step is one pass of the whole hot path over one decode token: kvs_decode_step, i.e. block scoring,
top-k and sparse attention:
  * 128k-max / 128k-mean: InternLM2.5-7B-shaped layer, 32 query / 8 KV heads, d 128, 131,072 cached
    tokens, block 128, Max (or Mean) reps, SHARED selection, top-96, Initial 128, Local 4,096;
    one query = one step of one sequence.  The JSON line's `value` is 128k-max.
  * 1m: 32 such layers of 1,048,576 tokens each (128 GiB of K/V resident), Quest reps, SEPARATE,
    top-64; one query = one decode token through all 32 layers (32 kvs_decode_step calls).
  * 8k: 8 query / 8 KV heads, 8,192 tokens, Quest, SEPARATE, top-8, Local 1,024.
  * 32k: Llama-2-70B-shaped GQA, 64 query / 8 KV heads, 32,768 tokens, Quest, SEPARATE, top-32.
  * mixed: 16 sequences of U[16K, 128K] tokens in one shuffled paged pool, Fix reps (every 16th
    token), SHARED, top-32, Local 2,048; each step builds the reps of the blocks that fill at it, then
    decodes the batch (16 queries per step).
  * the rows beyond the core path: Dynamic reps, preselect, Q8_0 / Q4_0 / INT8 caches.
Inputs are seeded synthetic fp16 (kvsynth) and resident in HBM before timing.  To keep repeated
steps from being served by the 256 MB Infinity Cache, a 128K step cycles through 16 cache replicas
(1.1 GB); a 1M step touches 2.7 GB of distinct memory anyway.  Steps are captured into HIP graphs
and replayed.

Roofline: algorithmic bytes per step = q + reps of every candidate block + K and V of every attended
token of every KV head + out, over the step time, against 8 TB/s.  The unit is one kvs_decode_step
call (its three or four kernels); profiles/ holds the per-kernel rocprofv3 averages of the same command.
traffic: HBM bytes per step from rocprofv3 FETCH_SIZE / WRITE_SIZE (profiles/), each scaled by what
the counter reads for the 4 GiB device copy timed at the start of every run; null when the kernels'
sources changed since the counters were taken.
cpu_baseline: the fp64 CPU oracle on the same inputs, reps prebuilt, on one thread and on one
single-threaded process per host core (up to 16), each for a bounded time.

Timing: every workload runs `--trials` timed runs of exactly `--steps` steps (the batched mixed
workload: whole windows of 128 steps), each bracketed by device synchronisations and HIP events; the
median run is reported with the fastest and slowest.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
B = 128
D = 128


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------------------------------------
# Workloads
# ------------------------------------------------------------------------------------------------
WORKLOADS = {
    "128k-max": dict(L=131072, Hq=32, Hkv=8, I=128, W=4096, k=96, rep="max", mode="shared",
                     layers=1, replicas=16, n_hot=50, hot_per_head=False, seed=20260002),
    "128k-mean": dict(L=131072, Hq=32, Hkv=8, I=128, W=4096, k=96, rep="mean", mode="shared",
                      layers=1, replicas=16, n_hot=50, hot_per_head=False, seed=20260012),
    "1m": dict(L=1 << 20, Hq=32, Hkv=8, I=128, W=4096, k=64, rep="quest", mode="separate",
               layers=32, replicas=1, n_hot=16, hot_per_head=True, seed=20260003),
    # 8K tokens, 8 query / 8 KV heads, 4 hot blocks shared by the heads
    "8k": dict(L=8192, Hq=8, Hkv=8, I=128, W=1024, k=8, rep="quest", mode="separate",
               layers=1, replicas=40, n_hot=4, hot_per_head=False, seed=20260000),
    # Llama-2-70B-shaped GQA: 64 query / 8 KV heads, 32K tokens, 8 hot blocks drawn per KV head
    "32k": dict(L=32768, Hq=64, Hkv=8, I=128, W=4096, k=32, rep="quest", mode="separate",
                layers=1, replicas=10, n_hot=8, hot_per_head=True, seed=20260001),
    # 16 sequences of U[16K, 128K] tokens in one shuffled paged pool (two pools alternate), Fix reps
    # every 16th token, SHARED, k 32, Local 2048: a window of 128 decode steps, each building the reps
    # of the blocks that fill at that step, then the batched decode step
    "mixed": dict(batch=16, Lmin=16384, Lmax=131072, Hq=32, Hkv=8, I=128, W=2048, k=32, rep="fix",
                  rep_num=8, mode="shared", layers=1, replicas=2, window=128, n_hot=8,
                  hot_per_head=False, seed=20260004),
    # the article's base configuration: Dynamic reps, one per block, from 32 observation queries
    "128k-dynamic": dict(L=131072, Hq=32, Hkv=8, I=128, W=4096, k=96, rep="dynamic", rep_num=1,
                         n_obs=32, mode="shared", layers=1, replicas=16, n_hot=50, hot_per_head=False,
                         seed=20260022),
    # selection confined to a preselected set of 192 blocks (token scores of 32 observation queries)
    "128k-presel": dict(L=131072, Hq=32, Hkv=8, I=128, W=4096, k=96, rep="max", mode="shared",
                        n_obs=32, presel=192, layers=1, replicas=16, n_hot=50, hot_per_head=False,
                        seed=20260032),
    # the same, with the set from pooled votes (average over a centred window of 7 tokens)
    "128k-presel-pool": dict(L=131072, Hq=32, Hkv=8, I=128, W=4096, k=96, rep="max", mode="shared",
                             n_obs=32, presel=192, pool=7, layers=1, replicas=16, n_hot=50,
                             hot_per_head=False, seed=20260032),
    # the same two headline shapes over a Q8_0 cache (kv_type): int8 codes + fp16 scale per 32 channels
    "128k-max-q8": dict(L=131072, Hq=32, Hkv=8, I=128, W=4096, k=96, rep="max", mode="shared",
                        layers=1, replicas=16, n_hot=50, hot_per_head=False, seed=20260002, kv="q8_0"),
    "1m-q8": dict(L=1 << 20, Hq=32, Hkv=8, I=128, W=4096, k=64, rep="quest", mode="separate",
                  layers=32, replicas=1, n_hot=16, hot_per_head=True, seed=20260003, kv="q8_0"),
    # and over a Q4_0 cache: 4-bit codes + fp16 scale per 32 channels
    "128k-max-q4": dict(L=131072, Hq=32, Hkv=8, I=128, W=4096, k=96, rep="max", mode="shared",
                        layers=1, replicas=16, n_hot=50, hot_per_head=False, seed=20260002, kv="q4_0"),
    "1m-q4": dict(L=1 << 20, Hq=32, Hkv=8, I=128, W=4096, k=64, rep="quest", mode="separate",
                  layers=32, replicas=1, n_hot=16, hot_per_head=True, seed=20260003, kv="q4_0"),
    # and over an INT8 cache with one fp32 scale per token and KV head
    "128k-max-i8": dict(L=131072, Hq=32, Hkv=8, I=128, W=4096, k=96, rep="max", mode="shared",
                        layers=1, replicas=16, n_hot=50, hot_per_head=False, seed=20260002, kv="int8_pth"),
    # and over an INT4 cache with one fp32 scale and one zero point per token and KV head
    "128k-max-i4": dict(L=131072, Hq=32, Hkv=8, I=128, W=4096, k=96, rep="max", mode="shared",
                        layers=1, replicas=16, n_hot=50, hot_per_head=False, seed=20260002, kv="int4_pth"),
}


def regions(L, I, W):
    ib = B * math.ceil(I / B)
    if L <= ib:
        return L, L, 0
    lloc = max(ib, B * math.floor((L - W) / B))
    return ib, lloc, (lloc - ib) // B


STEP_KERNELS = ("build_reps_kernel", "presel_step_kernel", "score_select_kernel", "score_kernel",
                "topk_il_wide_kernel", "topk_kernel", "attn_select_kernel", "merge_wave_kernel",
                "attn_tiles_kernel", "merge_kernel")
COPY_BYTES = 4 << 30  # the device copy of copy_bandwidth(): read and written once per dispatch


def source_hash() -> str:
    """sha256 over the HIP sources and the C header: the kernels the counters were taken on."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_sparse_kv_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc))
    for f in files + [os.path.join(ROOT, "include", "kvs.h")]:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_kv_file(path):
    """`key: value` lines of a profiles/ summary (other lines ignored)."""
    out = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.startswith((" ", "#", "|")):
                k, v = ln.split(":", 1)
                out[k.strip()] = v.strip()
    return out


def traffic_per_step(name):
    """HBM bytes per step from profiles/decode_step_<name>_traffic.txt, or None if absent or taken
    on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"decode_step_{name}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = read_kv_file(path)
    if kv.get("source_hash") != source_hash():
        return None
    return float(kv["hbm_bytes_per_step"])


def required_bytes(w, L=None):
    """Algorithmic bytes of one decode step of one layer of one sequence of L tokens."""
    L = w["L"] if L is None else L
    Hq, Hkv = w["Hq"], w["Hkv"]
    ie, ls, ncand = regions(L, w["I"], w["W"])
    k_eff = min(w["k"], ncand)
    T = min(ie, L) + k_eff * B + (L - ls)
    R = {"quest": 2, "max": 1, "mean": 1, "fix": w.get("rep_num", 1), "dynamic": w.get("rep_num", 1)}[w["rep"]]
    rep_elem = 4 if w["rep"] == "mean" else 2
    # bytes of one token's K (or V) row: fp16, or codes + one fp16 scale per 32 channels
    row = {"q8_0": D + (D // 32) * 2, "q4_0": D // 2 + (D // 32) * 2, "int8_pth": D + 4,
           "int4_pth": D // 2 + 4 + 1}.get(w.get("kv"), D * 2)
    return dict(q=Hq * D * 2, reps=ncand * Hkv * R * D * rep_elem, kv=Hkv * T * row * 2,
                out=Hq * D * 4, tokens=T, ncand=ncand, k_eff=k_eff)


class Setup:
    def __init__(self, name, device):
        import torch

        import block_sparse_kv_amd as kvs
        from block_sparse_kv_amd import ops
        import kvsynth

        w = WORKLOADS[name]
        self.name, self.w = name, w
        self.cfg = kvs.Config(num_q_heads=w["Hq"], num_kv_heads=w["Hkv"], initial_len=w["I"],
                              local_len=w["W"], topk=w["k"], rep_method=w["rep"],
                              rep_num=w.get("rep_num", 1), head_select_mode=w["mode"],
                              kv_type=w.get("kv", "fp16"))
        L = w["L"]
        nb = math.ceil(L / B)
        ie, ls, ncand = regions(L, w["I"], w["W"])
        lo, hi = ie // B, ie // B + ncand
        self.table = torch.arange(nb, dtype=torch.int32, device=device)[None]
        self.lens = torch.tensor([L], dtype=torch.int32, device=device)
        self.units = []  # one per (replica, layer): q, k_pool, v_pool, rep_pool
        self.presel = []  # per unit, with "presel" workloads: the preselected set
        n_units = w["replicas"] * w["layers"]
        t0 = time.time()
        for u in range(n_units):
            q, kp, vp, hot = kvsynth.pool_layer(kvsynth.mix_seed(w["seed"], u), L, w["Hq"], w["Hkv"],
                                                hot_range=(lo, hi), n_hot=w["n_hot"],
                                                hot_per_head=w["hot_per_head"], device=device)
            if w.get("kv", "fp16") != "fp16":  # quantized by the library; the fp16 tiles are dropped
                ids = torch.arange(nb, dtype=torch.int32)
                kp = ops.quantize_kv(self.cfg, kp, ids, ops.alloc_q8_pool(self.cfg, nb, device))
                vp = ops.quantize_kv(self.cfg, vp, ids, ops.alloc_q8_pool(self.cfg, nb, device))
            rp = ops.alloc_rep_pool(self.cfg, nb, device)
            if w["rep"] == "dynamic":  # token scores from the last n_obs queries, then the reps
                q_obs = kvsynth.randn_fp16((1, w["n_obs"], w["Hq"], D), kvsynth.mix_seed(w["seed"], u, 9), device)
                self.dyn = (q_obs, kp)
                imp = ops.token_importance(self.cfg, q_obs, kp, self.table, self.lens)
                ops.build_dynamic_reps(self.cfg, kp, imp, self.table, self.lens, rp)
            else:
                ops.build_reps(self.cfg, kp, torch.arange(L // B, dtype=torch.int32), rp)
            if "presel" in w:  # the unit's preselected set, from its own observation queries
                q_obs = kvsynth.randn_fp16((1, w["n_obs"], w["Hq"], D), kvsynth.mix_seed(w["seed"], u, 9), device)
                imp = ops.token_importance(self.cfg, q_obs, kp, self.table, self.lens)
                ps, _ = ops.preselect_blocks(self.cfg, imp, self.lens, w["presel"], nb, w.get("pool", 0))
                self.presel.append(ps)
                self.imp = imp
            self.units.append((q[None].contiguous(), kp, vp, rp))
        torch.cuda.synchronize()
        log(f"[setup] {name}: {n_units} cache units of {L} tokens generated in {time.time() - t0:.1f}s")
        self.out = torch.empty((1, w["Hq"], D), dtype=torch.float32, device=device)
        self.ws_bytes = kvs.kvs_decode_step_workspace_size(self.cfg, 1, nb)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=device)  # counters start at 0
        self.sel = torch.empty((1, self.cfg.groups, w["k"]), dtype=torch.int32, device=device)
        self.cnt = torch.empty((1, self.cfg.groups), dtype=torch.int32, device=device)
        self.nb = nb
        self.kvs = kvs
        if "presel" in w:
            self.pws_bytes = kvs.kvs_decode_step_preselected_workspace_size(self.cfg, 1, nb, w["presel"])
            self.pws = torch.zeros(self.pws_bytes, dtype=torch.uint8, device=device)  # counters start at 0

    @property
    def cycle(self):
        """Distinct step instances one captured cycle runs through (the cache replicas)."""
        return self.w["replicas"]

    def bulk_build(self, device, trials=6):
        """kvs_build_reps over every full block of replica 0 (layer 0): the post-prefill build."""
        import torch

        w = self.w
        _, kp, _, rp = self.units[0]
        nfull = w["L"] // B
        ids = torch.arange(nfull, dtype=torch.int32, device=device)
        times = []
        for _ in range(trials):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            self.kvs.kvs_build_reps(self.cfg, kp, ids, nfull, rp)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / 1e3)
        R = {"quest": 2, "max": 1, "mean": 1, "fix": w.get("rep_num", 1)}[w["rep"]]
        rep_row = D * (4 if w["rep"] == "mean" else 2)
        rd = nfull * w["Hkv"] * (B * D * 2 if w["rep"] != "fix" else R * D * 2)
        wr = nfull * w["Hkv"] * R * rep_row
        t = sorted(times[1:])[len(times[1:]) // 2]
        return dict(blocks=nfull, kv_heads=w["Hkv"], bytes_read=rd, bytes_written=wr, ms=t * 1e3,
                    hbm_gbs=(rd + wr) / t / 1e9, frac=(rd + wr) / t / 1e9 / PEAK_HBM_GBS)

    def step(self, replica):
        """One decode step (all layers) on cache replica `replica`."""
        w = self.w
        for layer in range(w["layers"]):
            self.step_unit(replica * w["layers"] + layer)

    def step_unit(self, u):
        """The decode step of one layer: cache unit u."""
        w = self.w
        q, kp, vp, rp = self.units[u]
        if self.presel:
            self.kvs.kvs_decode_step_preselected(self.cfg, q, kp, vp, rp, self.table, self.nb,
                                                 self.lens, 1, self.presel[u], w["presel"], self.out,
                                                 self.sel, self.cnt, self.pws, self.pws_bytes)
        else:
            self.kvs.kvs_decode_step(self.cfg, q, kp, vp, rp, self.table, self.nb, self.lens, 1,
                                     self.out, self.sel, self.cnt, self.ws, self.ws_bytes)

    def prepare_reuse(self):
        """Selection reuse (a later token or layer attends with an earlier selection): keep each
        unit's selection from one decode step, for attention-only steps."""
        import torch

        w = self.w
        self.reuse = []
        for u, (q, kp, vp, rp) in enumerate(self.units):
            sel = torch.empty_like(self.sel)
            cnt = torch.empty_like(self.cnt)
            self.kvs.kvs_decode_step(self.cfg, q, kp, vp, rp, self.table, self.nb, self.lens, 1,
                                     self.out, sel, cnt, self.ws, self.ws_bytes)
            self.reuse.append((sel, cnt))
        self.attn_ws_bytes = self.kvs.kvs_attn_workspace_size(self.cfg, 1, self.nb)
        self.attn_ws = torch.empty(self.attn_ws_bytes, dtype=torch.uint8, device=self.out.device)
        torch.cuda.synchronize()

    def step_attn(self, replica):
        """One attention-only step (all layers) with the kept selections."""
        w = self.w
        for layer in range(w["layers"]):
            u = replica * w["layers"] + layer
            q, kp, vp, _ = self.units[u]
            sel, cnt = self.reuse[u]
            self.kvs.kvs_sparse_decode_attn(self.cfg, q, kp, vp, self.table, self.nb, self.lens, 1,
                                            sel, cnt, self.out, self.attn_ws, self.attn_ws_bytes)


class MixedSetup:
    """The batched mixed-length workload: `batch` sequences of seeded U[Lmin, Lmax] tokens in one
    shuffled paged pool per replica (two replicas alternate step by step, so the 256 MB Infinity
    Cache does not serve a step from the one before).  A cycle is a window of `window` decode steps:
    at step t every sequence holds L_i + t tokens, the pools being filled to L_i + window beforehand;
    the step first builds the reps of the blocks that become full at t (one per sequence per 128
    steps), then runs kvs_decode_step on the whole batch."""

    def __init__(self, name, device):
        import torch

        import block_sparse_kv_amd as kvs
        from block_sparse_kv_amd import ops
        import kvsynth

        w = WORKLOADS[name]
        self.name, self.w, self.kvs = name, w, kvs
        self.cfg = kvs.Config(num_q_heads=w["Hq"], num_kv_heads=w["Hkv"], initial_len=w["I"],
                              local_len=w["W"], topk=w["k"], rep_method=w["rep"],
                              rep_num=w.get("rep_num", 1), head_select_mode=w["mode"])
        win, bsz = w["window"], w["batch"]
        self.lens0 = mixed_lengths(w)
        hot = []
        for L in self.lens0:
            ie, _, nc = regions(L, w["I"], w["W"])
            hot.append((ie // B, ie // B + nc))
        t0 = time.time()
        self.units = []
        for r in range(w["replicas"]):
            q, kp, vp, table, _ = kvsynth.pool_batch(kvsynth.mix_seed(w["seed"], 2, r),
                                                     [L + win for L in self.lens0], w["Hq"], w["Hkv"],
                                                     hot_ranges=hot, n_hot=w["n_hot"], device=device)
            rp = ops.alloc_rep_pool(self.cfg, kp.shape[0], device)
            full = torch.cat([table[i, : (L + win - 1) // B] for i, L in enumerate(self.lens0)])
            ops.build_reps(self.cfg, kp, full, rp)
            fill = []  # per window step: physical ids of the blocks that become full at that step
            for t in range(win):
                ids = [int(table[i, (L + t) // B - 1]) for i, L in enumerate(self.lens0) if (L + t) % B == 0]
                fill.append(torch.tensor(ids, dtype=torch.int32, device=device))
            self.units.append((q, kp, vp, rp, table, fill))
        torch.cuda.synchronize()
        log(f"[setup] {name}: {w['replicas']} pools of {bsz} sequences ({min(self.lens0)}..{max(self.lens0)} "
            f"tokens) generated in {time.time() - t0:.1f}s")
        self.nb = self.units[0][4].shape[1]
        self.lens_t = [torch.tensor([L + t for L in self.lens0], dtype=torch.int32, device=device)
                       for t in range(win)]
        self.out = torch.empty((bsz, w["Hq"], D), dtype=torch.float32, device=device)
        self.ws_bytes = kvs.kvs_decode_step_workspace_size(self.cfg, bsz, self.nb)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=device)  # counters start at 0
        self.sel = torch.empty((bsz, self.cfg.groups, w["k"]), dtype=torch.int32, device=device)
        self.cnt = torch.empty((bsz, self.cfg.groups), dtype=torch.int32, device=device)

    @property
    def cycle(self):
        return self.w["window"]

    def step(self, t):
        """Window step t: reps of the blocks filling at t, then one decode step of the batch."""
        q, kp, vp, rp, table, fill = self.units[t % self.w["replicas"]]
        ids = fill[t]
        if ids.numel():
            self.kvs.kvs_build_reps(self.cfg, kp, ids, ids.numel(), rp)
        self.kvs.kvs_decode_step(self.cfg, q, kp, vp, rp, table, self.nb, self.lens_t[t], self.w["batch"],
                                 self.out, self.sel, self.cnt, self.ws, self.ws_bytes)

    def window_bytes(self):
        return mixed_window_bytes(self.w, self.lens0)


def mixed_lengths(w):
    """The batched workload's starting lengths (seeded, CPU)."""
    import kvsynth

    return kvsynth.uniform_lengths(kvsynth.mix_seed(w["seed"], 1), w["batch"], w["Lmin"], w["Lmax"])


def mixed_window_bytes(w, lens0):
    """Algorithmic bytes of one window of the batched workload: every step's decode bytes, plus the
    rows of the reps built (read and written)."""
    tot = 0
    R = w.get("rep_num", 1)
    for t in range(w["window"]):
        for L in lens0:
            rb = required_bytes(w, L + t)
            tot += rb["q"] + rb["reps"] + rb["kv"] + rb["out"]
        n_fill = sum(1 for L in lens0 if (L + t) % B == 0)
        tot += n_fill * w["Hkv"] * R * D * 2 * 2
    return tot


def required_per_step(name):
    """Algorithmic bytes of one step of `name` (every layer; the batched workload: a window's mean)."""
    w = WORKLOADS[name]
    if "batch" in w:
        return mixed_window_bytes(w, mixed_lengths(w)) / w["window"]
    rb = required_bytes(w)
    return (rb["q"] + rb["reps"] + rb["kv"] + rb["out"]) * w["layers"]


def _capture(step_fn, idxs):
    import torch

    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in idxs:
            step_fn(i)
    g.replay()
    torch.cuda.synchronize()
    return g


def time_steps(setup, steps, warmup, trials=7, step_fn=None, whole_cycles=False):
    """Times `trials` runs of exactly `steps` steps (whole cycles when whole_cycles: at least `steps`)
    replayed from HIP graphs: a cycle (one step per replica, in order) and, when `steps` is not a
    multiple of it, a graph of the cycle's first `steps % cycle` steps.  Returns (list of seconds per
    run, steps per run, graph used?).  step_fn(i) defaults to the decode step of cycle position i."""
    import torch

    step_fn = step_fn or setup.step
    C = setup.cycle
    if whole_cycles:
        steps = max(C, -(-steps // C) * C)
    for i in range(warmup):
        step_fn(i % C)
    torch.cuda.synchronize()
    full = part = None
    graphed = True
    try:
        full = _capture(step_fn, range(C)) if steps >= C else None
        part = _capture(step_fn, range(steps % C)) if steps % C else None
    except Exception as e:  # capture unsupported: time eager launches instead
        log(f"[bench] graph capture failed ({e}); timing eager launches")
        graphed = False
    times = []
    for _ in range(trials):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        if graphed:
            for _ in range(steps // C):
                full.replay()
            if part is not None:
                part.replay()
        else:
            for i in range(steps):
                step_fn(i % C)
        end.record()
        torch.cuda.synchronize()
        times.append(start.elapsed_time(end) / 1e3)
    return times, steps, graphed


def copy_bandwidth(device, nbytes=4 << 30):
    import torch

    a = torch.empty(nbytes // 2, dtype=torch.float16, device=device)
    b = torch.empty_like(a)
    a.fill_(1.0)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 10
    e0.record()
    for _ in range(n):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3
    del a, b
    return 2.0 * nbytes * n / sec / 1e9


def _cpu_worker(args):
    """One process of the CPU baseline: the oracle's decode step on the saved inputs, repeated for
    `budget_s` seconds with one BLAS thread; returns the number of steps done."""
    d, kw, budget_s = args
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import kvs_oracle as orc

    q = np.load(os.path.join(d, "q.npy"))
    K = np.load(os.path.join(d, "K.npy"), mmap_mode="r")
    V = np.load(os.path.join(d, "V.npy"), mmap_mode="r")
    reps = np.load(os.path.join(d, "reps.npy"))
    n, t0 = 0, time.time()
    with threadpool_limits(limits=1):
        while True:
            orc.decode_step(q, K, V, reps=reps, **kw)
            n += 1
            if time.time() - t0 > budget_s:
                break
    return n, time.time() - t0


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(setup, budget_s=12.0, max_workers=16):
    """The fp64 oracle on replica 0 / layer 0 of the same inputs (reps prebuilt), untuned: one
    process with one thread, then one single-threaded process per host core (up to the box's share
    of 16), each running whole decode steps; queries/s = steps done / wall time / layers."""
    import multiprocessing as mp
    import shutil
    import tempfile

    import numpy as np

    import kvsynth
    from oracle import kvs_oracle as orc

    w = setup.w
    q, kp, vp, _ = setup.units[0]
    L = w["L"]
    d = tempfile.mkdtemp(prefix="kvs_cpu_")
    try:
        K = kvsynth.logical_from_pool(kp, setup.table[0].cpu(), L).cpu().numpy()
        np.save(os.path.join(d, "K.npy"), K)
        np.save(os.path.join(d, "V.npy"), kvsynth.logical_from_pool(vp, setup.table[0].cpu(), L).cpu().numpy())
        np.save(os.path.join(d, "q.npy"), q[0].cpu().numpy())
        _, _, cand = orc.regions(L, B, w["I"], w["W"])
        np.save(os.path.join(d, "reps.npy"), orc.block_reps(K, B, w["rep"], 1, blocks=cand))
        del K
        kw = dict(B=B, initial_len=w["I"], local_len=w["W"], topk=w["k"], method=w["rep"], mode=w["mode"])
        n1, t1 = _cpu_worker((d, kw, budget_s))
        avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
        workers = max(1, min(max_workers, avail))
        ctx = mp.get_context("spawn")  # fresh interpreters: nothing of this process's GPU state
        t0 = time.time()
        with ctx.Pool(workers) as pool:
            res = pool.map(_cpu_worker, [(d, kw, budget_s)] * workers)
        wall = time.time() - t0
    finally:
        shutil.rmtree(d, ignore_errors=True)
    n_all = sum(r[0] for r in res)
    qps1 = n1 / t1 / w["layers"]
    qps_all = sum(r[0] / r[1] for r in res) / w["layers"]  # the processes ran concurrently
    return dict(value=qps_all, unit="queries/s", cores=workers, kind="oracle",
                one_thread=dict(value=qps1, cores=1, steps=n1, seconds=t1),
                all_cores=dict(value=qps_all, cores=workers, steps=n_all, seconds=wall),
                nproc=os.cpu_count(), cpu_model=_cpu_model(),
                sample=f"single-layer decode steps of {setup.name} (replica 0, layer 0; reps prebuilt), "
                       f"fp64 numpy oracle, ~{budget_s:.0f} s per process: 1 process x 1 thread "
                       f"({n1} steps), then {workers} single-threaded processes at once ({n_all} steps); "
                       f"queries/s = sum of each process's steps / its time / {w['layers']} layers")


def _stats(times, steps):
    per = sorted(t / steps for t in times)
    return per[len(per) // 2], per[0], per[-1]


def measure(name, steps, warmup, device, trials=7, reuse=True):
    import torch

    w = WORKLOADS[name]
    mixed = "batch" in w
    st = MixedSetup(name, device) if mixed else Setup(name, device)
    times, steps_done, graphed = time_steps(st, steps, warmup, trials, whole_cycles=mixed)
    step_s, step_lo, step_hi = _stats(times, steps_done)
    if mixed:
        per_step = st.window_bytes() / w["window"]
        per_layer = per_step
        qn = w["batch"]
        rbs = [required_bytes(w, L) for L in st.lens0]
        extra = dict(batch=qn, lengths=st.lens0, window=w["window"],
                     attended_tokens_mean=sum(r["tokens"] for r in rbs) / qn,
                     candidates_mean=sum(r["ncand"] for r in rbs) / qn, k_eff=min(r["k_eff"] for r in rbs))
    else:
        rb = required_bytes(w)
        per_layer = rb["q"] + rb["reps"] + rb["kv"] + rb["out"]
        per_step = per_layer * w["layers"]
        qn = 1
        extra = dict(attended_tokens=rb["tokens"], candidates=rb["ncand"], k_eff=rb["k_eff"])
    gbs = per_step / step_s / 1e9
    res = dict(workload=name, steps=steps_done, trials=trials, graph=graphed, ms_per_step=step_s * 1e3,
               ms_per_step_min=step_lo * 1e3, ms_per_step_max=step_hi * 1e3, queries_per_step=qn,
               queries_per_s=qn / step_s, required_bytes_per_step=per_step,
               required_bytes_per_layer=per_layer, hbm_gbs=gbs, frac=gbs / PEAK_HBM_GBS,
               traffic_bytes_per_step=traffic_per_step(name), **extra, setup=st)
    log(f"[bench] {name}: {step_s * 1e6:.1f} us/step (min {step_lo * 1e6:.1f}, max {step_hi * 1e6:.1f}, "
        f"{trials} runs of {steps_done} steps), {qn / step_s:.0f} queries/s, {gbs:.0f} GB/s = "
        f"{100 * gbs / PEAK_HBM_GBS:.1f}% of 8 TB/s (graph={graphed})")
    if not mixed and "kv" not in w and w["rep"] != "dynamic" and "presel" not in w:
        res["bulk_build_reps"] = bb = st.bulk_build(device)
        log(f"[bench] {name} kvs_build_reps over {bb['blocks']} blocks x {bb['kv_heads']} KV heads: "
            f"{bb['ms']:.3f} ms, {bb['hbm_gbs']:.0f} GB/s = {100 * bb['frac']:.1f}% of 8 TB/s")
    if w["rep"] == "dynamic":  # the per-prompt cost of Dynamic reps: token scores + reps of one cache
        from block_sparse_kv_amd import ops
        q_obs, kp = st.dyn
        rp = ops.alloc_rep_pool(st.cfg, st.nb, device)
        times = []
        for _ in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            imp = ops.token_importance(st.cfg, q_obs, kp, st.table, st.lens)
            ops.build_dynamic_reps(st.cfg, kp, imp, st.table, st.lens, rp)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        kbytes = 2 * w["Hkv"] * w["L"] * D * 2  # K read by both passes over the scores
        res["dynamic_reps_build"] = dict(ms=min(times[1:]), n_obs=w["n_obs"], k_bytes_read=kbytes,
                                         hbm_gbs=kbytes / (min(times[1:]) * 1e-3) / 1e9)
        log(f"[bench] {name} token scores + Dynamic reps of one {w['L']}-token cache: "
            f"{min(times[1:]):.3f} ms ({kbytes / (min(times[1:]) * 1e-3) / 1e9:.0f} GB/s on K)")
    if "presel" in w:  # the per-prompt cost of the set: block scores + top-k over one cache's scores
        from block_sparse_kv_amd import ops
        times = []
        for _ in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            ops.preselect_blocks(st.cfg, st.imp, st.lens, w["presel"], st.nb, w.get("pool", 0))
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        res["preselect_build"] = dict(ms=min(times[1:]), pool_kernel=w.get("pool", 0), n_presel=w["presel"])
        log(f"[bench] {name} preselected set of one {w['L']}-token cache from its token scores: "
            f"{min(times[1:]):.3f} ms (pool_kernel {w.get('pool', 0)})")
    if not reuse or mixed:
        return res
    # selection reuse: attention only, with each unit's kept selection (no scoring, no top-k)
    st.prepare_reuse()
    times_a, steps_a, _ = time_steps(st, steps, warmup, trials, step_fn=st.step_attn)
    attn_s, _, _ = _stats(times_a, steps_a)
    rb = required_bytes(w)
    attn_bytes = (rb["q"] + rb["kv"] + rb["out"]) * w["layers"]
    res["reuse_attention_only"] = dict(ms_per_step=attn_s * 1e3, queries_per_s=1.0 / attn_s,
                                       required_bytes_per_step=attn_bytes,
                                       hbm_gbs=attn_bytes / attn_s / 1e9,
                                       frac=attn_bytes / attn_s / 1e9 / PEAK_HBM_GBS)
    log(f"[bench] {name} attention only (selection reused): {attn_s * 1e6:.1f} us/step, "
        f"{attn_bytes / attn_s / 1e9:.0f} GB/s = {100 * attn_bytes / attn_s / 1e9 / PEAK_HBM_GBS:.1f}%")
    if "kv" not in w:
        res["gather_reference"] = g = gather_reference(st, device)
        log(f"[bench] {name} plain gather of one layer's attended tiles (torch index_select of K and V, "
            f"{g['tiles']} tiles each, cycling over {g['units']} cache units): {g['us']:.1f} us, "
            f"{g['bytes_read'] / 1e6:.1f} MB read and as much written, {g['read_gbs']:.0f} GB/s read")
        log(f"[bench] {name} read floor of the same tiles (kvs_gather_read_floor, reads and sums only): "
            f"{g['floor_us']:.1f} us = {g['floor_read_gbs']:.0f} GB/s; with 36,864 B of LDS per "
            f"workgroup as the attention tiles: {g['floor_tile_lds_us']:.1f} us = "
            f"{g['floor_tile_lds_read_gbs']:.0f} GB/s")
    return res


def gather_reference(st, device, replays=20):
    """A library gather of the tiles one layer's decode step attends (unit 0's Initial/Local tiles
    and the selection kept by prepare_reuse), K and V, by torch.index_select into fresh buffers:
    what a plain copy of the same scattered 32 KiB tiles costs on this part, for comparison with the
    attention launch that reads them.  Then the read floor of the same tiles: the library's
    read-only kernel (kvs_gather_read_floor), with no LDS reserved and with an attention tile's.
    Each is captured once per cache unit (the same tile ids in every unit's pools, as the timed
    steps cycle over the units, so the reads are not served from a cache), graph-replayed; the
    median replay over the number of units."""
    import torch
    from block_sparse_kv_amd import binding

    w = st.w
    Hkv = w["Hkv"]
    ie, ls, _ = regions(w["L"], w["I"], w["W"])
    il = list(range(ie // B)) + list(range(ls // B, (w["L"] + B - 1) // B))
    sel, cnt = st.reuse[0]
    sel, cnt, table = sel.cpu().numpy(), cnt.cpu().numpy(), st.table.cpu().numpy()
    idx = []
    for h in range(Hkv):
        gi = h if st.cfg.groups == Hkv else 0
        blocks = il + [int(b) for b in sel[0, gi, : int(cnt[0, gi])]]
        idx += [int(table[0, b]) * Hkv + h for b in blocks]  # (physical block, KV head) tile
    ix = torch.tensor(idx, dtype=torch.long, device=device)
    ix32 = ix.to(torch.int32)
    pools = [(kp, vp) for _, kp, vp, _ in st.units]
    ko = torch.empty((len(idx), B * D), dtype=pools[0][0].dtype, device=device)
    vo = torch.empty_like(ko)
    sums = torch.empty(len(idx), dtype=torch.float32, device=device)

    def copy(u):
        kp, vp = pools[u]
        torch.index_select(kp.view(-1, B * D), 0, ix, out=ko)
        torch.index_select(vp.view(-1, B * D), 0, ix, out=vo)

    def floor(lds):
        def run(u):
            kp, vp = pools[u]
            binding.kvs_gather_read_floor(kp, vp, kp.numel() // (B * D), ix32, len(idx), lds, sums)
        return run

    def timed(fn):
        for u in range(len(pools)):
            fn(u)
        torch.cuda.synchronize()
        g = _capture(fn, range(len(pools)))
        times = []
        for _ in range(replays):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3 / len(pools))
        return sorted(times)[len(times) // 2]

    nbytes = 2 * len(idx) * B * D * 2
    t = timed(copy)
    res = dict(tiles=len(idx), units=len(pools), us=t * 1e6, bytes_read=nbytes, read_gbs=nbytes / t / 1e9)
    for lds, key in ((0, "floor"), (36864, "floor_tile_lds")):
        tf = timed(floor(lds))
        res[key + "_us"] = tf * 1e6
        res[key + "_read_gbs"] = nbytes / tf / 1e9
    return res


# ------------------------------------------------------------------------------------------------
# rocprofv3 output -> profiles/ summaries
# ------------------------------------------------------------------------------------------------
def _step_kernel(name):
    base = name.split("(")[0].split("<")[0].replace("void ", "").strip()
    return base.replace("kvs::", "") if base.replace("kvs::", "") in STEP_KERNELS else None


def _bench_line(log_path):
    if log_path and os.path.exists(log_path):
        with open(log_path) as f:
            for ln in f:
                if ln.startswith("[bench]") and "us/step" in ln:
                    return ln.strip()
    return "(bench log not given)"


def summarize_stats(d, name, log_path=None, steps=480, out_dir=None):
    """rocprofv3 --kernel-trace --stats CSV -> profiles/decode_step_<name>_kernel_stats.txt."""
    import csv

    rows = [r for r in csv.DictReader(open(os.path.join(d, "run_kernel_stats.csv")))
            if _step_kernel(r["Name"]) is not None]
    # kernels called at least half as often as the busiest one run every layer step; the others
    # (the set-up's rep builds and preselection, the batched workload's incremental builds) do not
    top = max(int(r["Calls"]) for r in rows)
    out, tot = [], 0.0
    for r in rows:
        k = _step_kernel(r["Name"])
        avg = float(r["AverageNs"]) / 1e3
        every = int(r["Calls"]) >= top // 2
        if every:
            tot += avg
        out.append(f"| {k + ('' if every else ' *'):20s} | {r['Name'][:60]:60s} | {int(r['Calls']):6d} | "
                   f"{avg:9.2f} | {float(r['MinNs']) / 1e3:9.2f} | {float(r['MaxNs']) / 1e3:9.2f} |")
    txt = [f"# kvs_decode_step kernels, workload {name}",
           "",
           "command (repository root on the MI355X box; bench.py times the same calls):",
           f"    rocprofv3 --kernel-trace --stats --output-format csv -d {d} -o run "
           f"-- python3 bench.py --workload {name} --no-cpu --no-reuse --steps {steps}"
           + (f" > {log_path} 2>&1" if log_path else ""),
           f"    python bench.py --summarize-stats {d} --workload {name} --steps {steps}"
           + (f" --log {log_path}" if log_path else ""),
           "",
           f"source_hash: {source_hash()}",
           f"sum_of_kernel_averages_us_per_layer: {tot:.2f}",
           f"bench_line_under_the_profiler: {_bench_line(log_path)}",
           "",
           "| kernel               | name                                                         |  calls |  avg us   |  min us   |  max us   |",
           "|----------------------|--------------------------------------------------------------|--------|-----------|-----------|-----------|",
           *out,
           "",
           "* not every layer step (set-up, or the batched workload's incremental rep builds): not in the sum",
           ""]
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"decode_step_{name}_kernel_stats.txt")
    with open(path, "w") as f:
        f.write("\n".join(txt))
    print(path)


def summarize_pmc(fetch_dir, write_dir, name, steps=32, out_dir=None):
    """rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs -> profiles/decode_step_<name>_traffic.txt.
    Each counter is scaled by what it reads for the 4 GiB copies of copy_bandwidth().  Per layer:
    the mean bytes per dispatch of each decode-step kernel, summed (the batched workload's
    incremental rep builds, not run every step, are listed but not summed)."""
    import csv
    import collections

    w = WORKLOADS[name]
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = collections.defaultdict(list)
        copies = []
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"]) * 1024.0  # KiB per dispatch
            if "copyBuffer" in r["Kernel_Name"]:
                copies.append(v)
            k = _step_kernel(r["Kernel_Name"])
            if k is not None:
                per[k].append(v)
        big = max(copies)
        cal = [v for v in copies if v >= 0.5 * big]  # the 4 GiB copies
        scale = COPY_BYTES / (sum(cal) / len(cal))
        res[counter] = (scale, {k: sum(v) / len(v) * scale for k, v in per.items()},
                        {k: len(v) for k, v in per.items()}, len(cal))
    # as in summarize_stats: kernels dispatched at least half as often as the busiest run every step
    top = max(res["FETCH_SIZE"][2].values())
    every = {k for k, n in res["FETCH_SIZE"][2].items() if n >= top // 2}
    req_layer = required_per_step(name) / w["layers"]
    fetch_layer = sum(v for k, v in res["FETCH_SIZE"][1].items() if k in every)
    write_layer = sum(v for k, v in res["WRITE_SIZE"][1].items() if k in every)
    lines = [f"# HBM traffic of kvs_decode_step, workload {name}",
             "",
             "commands (repository root on the MI355X box), one counter per run:",
             f"    rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o run "
             f"-- python3 bench.py --workload {name} --no-cpu --no-reuse --steps {steps} --warmup 2",
             f"    rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o run "
             f"-- python3 bench.py --workload {name} --no-cpu --no-reuse --steps {steps} --warmup 2",
             f"    python bench.py --summarize-pmc {fetch_dir} {write_dir} --workload {name} --steps {steps}",
             "",
             "Calibration: each counter over the 4 GiB device copy that starts every bench.py run "
             "(read 4 GiB, write 4 GiB).",
             f"fetch_scale: {res['FETCH_SIZE'][0]:.4f}",
             f"write_scale: {res['WRITE_SIZE'][0]:.4f}",
             f"source_hash: {source_hash()}",
             f"required_bytes_per_layer: {req_layer}",
             f"fetch_bytes_per_layer: {fetch_layer:.0f}",
             f"write_bytes_per_layer: {write_layer:.0f}",
             f"hbm_bytes_per_step: {(fetch_layer + write_layer) * w['layers']:.0f}",
             f"traffic_over_required: {(fetch_layer + write_layer) / req_layer:.4f}",
             "",
             "| kernel               | dispatches | fetch bytes (scaled) | write bytes (scaled) |",
             "|----------------------|------------|----------------------|----------------------|"]
    for k in STEP_KERNELS:
        if k in res["FETCH_SIZE"][1]:
            lines.append(f"| {k + ('' if k in every else ' *'):20s} | {res['FETCH_SIZE'][2][k]:10d} | "
                         f"{res['FETCH_SIZE'][1][k]:20.0f} | {res['WRITE_SIZE'][1].get(k, 0.0):20.0f} |")
    lines += ["", "* not every layer step (set-up, or the batched workload's incremental rep builds): "
              "not in the per-layer sums"]
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"decode_step_{name}_traffic.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)


TL_KINDS = ("scoring+selection: scoring workgroups", "scoring+selection: Initial/Local tiles",
            "top-k launch: Initial/Local tiles", "attention: selected tiles", "merge",
            "top-k launch: selections", "scoring launch", "top-k launch (own)", "compaction", "map back",
            "attention: selections by the tiles", "attention: Initial/Local tiles")
TL_LAUNCH = {0: "scoring+selection", 1: "scoring+selection", 2: "top-k", 5: "top-k", 3: "attention",
             4: "merge", 6: "scoring", 7: "top-k (own)", 8: "compaction", 9: "map back", 10: "attention",
             11: "attention"}
TL_MARKS = {1: "operands in / scores stored", 2: "done / counter bumped", 3: "selection stored",
            4: "chunk summary stored", 5: "chunk summary made"}
TL_MAX_WG, TL_SLOTS = 16384, 8


def timeline_replay_stats(rec):
    """One replay's records [kinds][TL_MAX_WG][TL_SLOTS] (float64 ticks of the 100 MHz clock) ->
    {(kind, "n"): workgroups, (kind, slot): (min, median, max) us, (kind, "end"): last mark us}, times
    from the step's first scoring workgroup start.  The step starts with its scoring workgroups (first
    in their launch's grid, kinds 0 and 6); a record that starts earlier than 1 us before them is an
    earlier step's, left by a workgroup that had nothing to do this time, and is dropped."""
    import numpy as np

    first = [rec[k][rec[k][:, 0] > 0, 0].min() for k in (0, 6) if (rec[k][:, 0] > 0).any()]
    t_first = min(first)
    vals = {}
    for k in range(rec.shape[0]):
        r = rec[k][rec[k][:, 0] >= t_first - 100.0]
        if not len(r):
            continue
        vals[(k, "n")] = len(r)
        us = lambda a: (a - t_first) / 100.0
        for slot in (0, 1, 2, 3, 4, 5):
            a = r[:, slot]
            a = a[a > 0]
            if len(a):
                vals[(k, slot)] = (us(a.min()), us(np.median(a)), us(a.max()))
        marks = r[:, 1:6]
        vals[(k, "end")] = us(marks[marks > 0].max()) if (marks > 0).any() else us(r[:, 0].max())
    return vals


def timeline_medians(per_replay):
    """The median over replays of every figure present in all of them."""
    import statistics

    keys = [k for k in per_replay[-1] if all(k in v for v in per_replay)]
    med = {}
    for key in keys:
        xs = [v[key] for v in per_replay]
        med[key] = tuple(statistics.median(x[i] for x in xs) for i in range(3)) if isinstance(xs[0], tuple) \
            else statistics.median(xs)
    return med


def timeline_lines(med):
    """Text tables of timeline_medians(): per workgroup kind, then per launch (kinds grouped by
    TL_LAUNCH) with its first start, last mark, span and the gap after the launch before."""
    f3 = lambda t: f"{t[0]:6.2f} {t[1]:6.2f} {t[2]:6.2f}"
    lines = ["# workgroup kinds: start and marks, us from the layer's first workgroup start (min / median / max)"]
    kinds = sorted({k for k, _ in med}, key=lambda k: med[(k, 0)][0])
    for k in kinds:
        lines.append(f"| {TL_KINDS[k]:40s} | n {int(med[(k, 'n')]):5d} | start {f3(med[(k, 0)])} |")
        for slot in (1, 5, 4, 2, 3):
            if (k, slot) in med:
                lines.append(f"|   {TL_MARKS[slot]:38s} |         | {'':5s} {f3(med[(k, slot)])} |")
    lines += ["", "# launches: first workgroup start, last mark, span, gap after the launch before (us)"]
    launches = {}
    for k in kinds:
        L = TL_LAUNCH[k]
        s0, e0 = med[(k, 0)][0], med[(k, "end")]
        a, b = launches.get(L, (s0, e0))
        launches[L] = (min(a, s0), max(b, e0))
    prev_end = None
    for L, (a, b) in sorted(launches.items(), key=lambda x: x[1][0]):
        gap = f"{a - prev_end:6.2f}" if prev_end is not None else "     -"
        lines.append(f"| {L:20s} | start {a:6.2f} | end {b:6.2f} | span {b - a:6.2f} | gap {gap} |")
        prev_end = b
    lines.append(f"layer: {prev_end:.2f} us from the first workgroup start to the last mark "
                 "(the timeline build waits for loads at mark 1, so it runs a little slower than the default build)")
    return lines


def timeline(name, device, replays=9, keep=5):
    """Per-workgroup timeline of the last layer step of `name`'s timed cycle (the same graph-replayed
    cycle of steps over the cache replicas as the timed runs, so the layer's data is as cold as
    there), from the timeline library (KVS_LIBRARY=timeline): for each kind of workgroup its start
    and marks (min / median / max over workgroups, us from the layer's first workgroup start), and
    per launch its first start, last mark and the gap to the launch before.  Each figure is the
    median over the last `keep` of `replays` replays.  Returns the summary's text lines."""
    import numpy as np
    import torch

    import block_sparse_kv_amd as kvs
    from block_sparse_kv_amd import binding

    if not binding.TIMELINE:
        raise SystemExit("--timeline needs the timeline library: python block_sparse_kv_amd/build.py "
                         "--timeline, then KVS_LIBRARY=timeline python bench.py --timeline ...")
    n_kinds = len(TL_KINDS)
    buf = torch.zeros(n_kinds * TL_MAX_WG * TL_SLOTS, dtype=torch.int64, device=device)
    kvs.kvs_timeline_set(buf)  # read by every later call's configuration
    mixed = "batch" in WORKLOADS[name]
    st = MixedSetup(name, device) if mixed else Setup(name, device)
    for i in range(st.cycle):
        st.step(i)
    torch.cuda.synchronize()
    g = _capture(st.step, range(st.cycle))
    per_replay = []
    for _ in range(replays):
        buf.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        rec = buf.view(n_kinds, TL_MAX_WG, TL_SLOTS).cpu().numpy().view(np.uint64).astype(np.float64)
        per_replay.append(timeline_replay_stats(rec))
    kvs.kvs_timeline_set(None)
    med = timeline_medians(per_replay[-keep:])
    head = [f"workload: {name}",
            f"layer_step: the last {'batch step' if mixed else 'layer step'} of a graph-replayed cycle of "
            f"{st.cycle} steps ({WORKLOADS[name]['layers']} layers each), as in the timed runs",
            f"replays: {replays} (medians over the last {keep})",
            f"source_hash: {source_hash()}",
            "command: python block_sparse_kv_amd/build.py --timeline && "
            f"KVS_LIBRARY=timeline python bench.py --timeline {name}",
            ""]
    return head + timeline_lines(med)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=480)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--trials", type=int, default=7, help="timed runs of exactly --steps steps; the median is reported")
    ap.add_argument("--workload", default="all", choices=["all", *WORKLOADS])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-reuse", action="store_true",
                    help="skip the attention-only (reused selection) timing, e.g. under the profiler")
    ap.add_argument("--summarize-stats", metavar="DIR", help="rocprofv3 --stats output -> profiles/")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE outputs -> profiles/")
    ap.add_argument("--log", help="bench output captured under the profiler (for --summarize-stats)")
    ap.add_argument("--timeline", metavar="WORKLOAD", choices=list(WORKLOADS),
                    help="per-workgroup timeline of one layer's step (timeline library) -> profiles/")
    args = ap.parse_args()
    if args.timeline:
        lines = timeline(args.timeline, "cuda:0")
        path = os.path.join(ROOT, "profiles", f"decode_step_{args.timeline}_timeline.txt")
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        print("\n".join(lines))
        print(path)
        return
    if args.summarize_stats or args.summarize_pmc:
        if args.workload == "all":
            ap.error("--summarize-* needs --workload")
        if args.summarize_stats:
            summarize_stats(args.summarize_stats, args.workload, args.log, args.steps)
        if args.summarize_pmc:
            summarize_pmc(*args.summarize_pmc, args.workload, args.steps)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the block-sparse decode path is built and timed on a "
              "single MI355X (sharding is design-only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    device = "cuda:0"
    torch.cuda.set_device(0)
    copy_gbs = copy_bandwidth(device)
    log(f"[bench] device copy bandwidth {copy_gbs:.0f} GB/s")
    if args.workload == "all":
        # the headline first, then the single-sequence 128K-and-shorter workloads, then the ones that
        # allocate and free ~130 GB (32-layer 1M caches, the batched pools): after those, the others
        # measure up to a microsecond slower in the same process
        big = [n for n in WORKLOADS if WORKLOADS[n]["layers"] > 1 or "batch" in WORKLOADS[n]]
        names = [n for n in WORKLOADS if n not in big] + big
    else:
        names = [args.workload]
    results = {}
    for n in names:
        st_steps = args.steps if (n == names[0] or WORKLOADS[n]["layers"] == 1) else max(16, args.steps // 8)
        results[n] = measure(n, st_steps, args.warmup, device, trials=args.trials, reuse=not args.no_reuse)
        if n != names[0]:
            del results[n]["setup"]
            torch.cuda.empty_cache()
    head = results[names[0]]
    cpu = None
    if not args.no_cpu and "batch" not in WORKLOADS[names[0]]:
        cpu = cpu_baseline(head["setup"])
        log(f"[bench] cpu oracle: {cpu['one_thread']['value']:.2f} queries/s on 1 thread, "
            f"{cpu['value']:.2f} on {cpu['cores']} processes ({cpu['cpu_model']}, nproc {cpu['nproc']})")
    del head["setup"]
    w = WORKLOADS[names[0]]
    line = {
        "metric": "sparse decode queries/s + achieved HBM GB/s (% roofline) at 128K and 1M ctx",
        "value": head["queries_per_s"],
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "trials": head["trials"],
        "ms_per_step_min": head["ms_per_step_min"],
        "ms_per_step_max": head["ms_per_step_max"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic (seeded N(0,1) fp16 K/V/q with planted hot blocks)",
        "config": {"workload": names[0],
                   "context": w["L"] if "L" in w else f"U[{w['Lmin']}, {w['Lmax']}] + window {w['window']}",
                   "batch": w.get("batch", 1), "layers": w["layers"],
                   "q_heads": w["Hq"], "kv_heads": w["Hkv"], "head_dim": D, "block_size": B,
                   "rep": w["rep"], "head_select_mode": w["mode"], "topk": w["k"],
                   "initial": w["I"], "local": w["W"], "replicas": w["replicas"]},
        "roofline": {"bound": "hbm", "achieved": head["hbm_gbs"], "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": head["frac"],
                     "traffic": traffic_per_step(names[0]),
                     "kernel": "kvs_decode_step (one call: its scoring, selection, tile and merge "
                               "launches)",
                     "bytes_per_launch": head["required_bytes_per_step"]},
        "cpu_baseline": cpu,
        "copy_gbs": copy_gbs,
        "frac_of_copy": head["hbm_gbs"] / copy_gbs,
        "source_hash": source_hash(),
        "workloads": {k: {kk: vv for kk, vv in v.items() if kk != "setup"}
                      for k, v in results.items()},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
