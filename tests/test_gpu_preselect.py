"""Preselect on the GPU against the oracle (needs an MI355X).

The set: blocks ranked by the sum of their tokens' scores, or by their best vote after pooling over a
window of tokens (token scores as in the Dynamic rep tests), checked like any selection (exact, or
inside the 1e-4 tie band).  The confined decode step:
given a set, only its blocks that are still candidates compete; the selection is checked against the
oracle on that restricted candidate list, and the output against the oracle's attention over the
GPU's selection.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("no GPU", allow_module_level=True)

import block_sparse_kv_amd as kvs  # noqa: E402
from block_sparse_kv_amd import ops  # noqa: E402

import kvsynth  # noqa: E402
from oracle import kvs_oracle as orc  # noqa: E402
from parity import ATOL_OUT, B, Case, check_selection, method_name  # noqa: E402

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def build_reps(case):
    c = case.cfg
    rp = ops.alloc_rep_pool(c, case.pb.k_pool.shape[0], DEV)
    ids = [int(x) for i, L in enumerate(case.lens) for x in case.table[i, : L // B]]
    if ids:
        ops.build_reps(c, case.k_pool, torch.tensor(ids, dtype=torch.int32), rp)
    return rp


PRE_CASES = [
    # (Hq, Hkv, mode, rep, n_obs, n_presel, lens, pool_kernel): 0 ranks block sums, an odd kernel
    # the blocks' best pooled votes
    (32, 8, "shared", "max", 16, 20, [6000, 9000], 0),
    (8, 2, "separate", "quest", 8, 12, [5000], 0),
    (16, 4, "separate", "mean", 4, 200, [3000], 0),      # n_presel > n_cand: every candidate
    (16, 2, "shared", "quest", 8, 64, [280000], 0),      # long rows
    (32, 8, "shared", "max", 16, 20, [6000, 9000], 7),
    (8, 2, "separate", "quest", 8, 12, [5000, 700], 1),  # 700: no candidates
    (16, 4, "separate", "mean", 4, 30, [3000], 127),     # the widest window
    (16, 2, "shared", "quest", 8, 64, [140000], 5),      # long rows
]


@pytest.mark.parametrize("idx", range(len(PRE_CASES)))
def test_preselect_blocks(idx):
    Hq, Hkv, mode, rep, n_obs, n_presel, lens, pk = PRE_CASES[idx]
    say(f"[case] preselect {Hq}x{Hkv} {mode} n_obs={n_obs} n_presel={n_presel} lens={lens} pool={pk}")
    c = kvs.Config(num_q_heads=Hq, num_kv_heads=Hkv, initial_len=128, local_len=1024, topk=8,
                   rep_method=rep, head_select_mode=mode)
    case = Case(c, lens, seed=kvsynth.mix_seed(601, idx), n_hot=3)
    pb = case.pb
    q_obs = kvsynth.randn_fp16((len(lens), n_obs, Hq, 128), kvsynth.mix_seed(602, idx), DEV)
    imp = ops.token_importance(c, q_obs, case.k_pool, pb.block_table, pb.seq_lens)
    presel, pcnt = ops.preselect_blocks(c, imp, pb.seq_lens, n_presel, pb.max_blocks, pk)
    torch.cuda.synchronize()
    for i, L in enumerate(lens):
        ref_imp = orc.token_importance(q_obs[i].cpu().numpy(), case.host[i][1], mode)
        rows, cand = orc.preselect_scores(ref_imp, L, B, c.initial_len, c.local_len, pk)
        for gi in range(c.groups):
            check_selection(presel[i, gi].cpu().numpy(), pcnt[i, gi].item(), rows[gi], cand, n_presel,
                            f"preselect seq {i} grp {gi}")


STEP_CASES = [
    # (Hq, Hkv, mode, rep, k, lens, kv, set size): sets of up to 1024 entries are scored and selected
    # from in one launch; larger ones through every candidate's score, compacted rows and the
    # ordinary top-k
    (32, 8, "shared", "max", 6, [6000, 9000], "fp16", 18),
    (8, 2, "separate", "quest", 4, [5000], "fp16", 18),
    (16, 4, "separate", "quest", 40, [3000], "fp16", 18),   # k >= the set: the set itself
    (32, 8, "shared", "max", 10, [7000], "q8_0", 18),
    (16, 2, "shared", "quest", 16, [280000], "fp16", 18),   # long rows
    (16, 4, "separate", "max", 30, [60000], "q4_0", 248),   # 254 entries: the one-launch path near its limit
    (16, 2, "shared", "quest", 50, [60000, 40000], "fp16", 300),
    (32, 8, "separate", "mean", 12, [20000], "int8_pth", 40),
    (16, 4, "separate", "quest", 24, [280000], "fp16", 1100),  # 1106 entries: compacted rows
    (32, 8, "shared", "fix", 20, [150000, 90000], "fp16", 1012),  # 1018 entries: one launch, near its limit
    (8, 8, "separate", "max", 7, [130000], "q8_0", 300),  # every KV head its own set, g = 1
    # batch * Hkv * k > 1024: the scoring launch's last workgroup of each row selects
    (32, 8, "shared", "max", 70, [60000, 40000], "fp16", 100),
]


@pytest.mark.parametrize("idx", range(len(STEP_CASES)))
def test_decode_step_preselected(idx):
    Hq, Hkv, mode, rep, k, lens, kv, n_pick = STEP_CASES[idx]
    say(f"[case] confined decode step {Hq}x{Hkv} {mode} {rep} k={k} lens={lens} kv={kv} set={n_pick}")
    c = kvs.Config(num_q_heads=Hq, num_kv_heads=Hkv, initial_len=128, local_len=1024, topk=k,
                   rep_method=rep, head_select_mode=mode, kv_type=kv)
    case = Case(c, lens, seed=kvsynth.mix_seed(603, idx), n_hot=3)
    pb = case.pb
    rp = build_reps(case)
    # a set per group: random candidate blocks, some Local and Initial blocks (no longer candidates)
    # and -1 padding, ascending
    g = np.random.default_rng(kvsynth.mix_seed(604, idx))
    n_presel = n_pick + 6
    presel = np.full((len(lens), c.groups, n_presel), -1, dtype=np.int32)
    sets = []
    for i, L in enumerate(lens):
        _, _, cand = orc.regions(L, B, c.initial_len, c.local_len)
        row_sets = []
        for gi in range(c.groups):
            picks = sorted(set(g.choice(cand, size=min(n_pick, len(cand)), replace=False).tolist())
                           | {0, (L - 1) // B})  # an Initial and a Local block
            presel[i, gi, : len(picks)] = picks
            row_sets.append(picks)
        sets.append(row_sets)
    out, sel, cnt = ops.decode_step_preselected(c, pb.q, case.k_pool, case.v_pool, rp, pb.block_table,
                                                pb.seq_lens, torch.tensor(presel, device=DEV))
    torch.cuda.synchronize()
    for i, L in enumerate(lens):
        ref = case.oracle(i)  # every candidate's score (reps as the rep pool stores them)
        cand = ref["cand"]
        pos = {b: j for j, b in enumerate(cand)}
        for gi in range(c.groups):
            allowed = [b for b in sets[i][gi] if b in pos]
            row = [ref["scores"][gi][pos[b]] for b in allowed]
            check_selection(sel[i, gi].cpu().numpy(), cnt[i, gi].item(), row, allowed, k,
                            f"confined sel seq {i} grp {gi}")
            if k >= len(allowed):
                assert [int(x) for x in sel[i, gi, : len(allowed)].cpu()] == allowed
        gsel = [[int(x) for x in sel[i, gi, : int(cnt[i, gi])].cpu()] for gi in range(c.groups)]
        err = case.check_out(out, i, case.oracle_attention(i, gsel), "confined decode step")
        say(f"[ok] seq {i}: max err {err:.2e}")
