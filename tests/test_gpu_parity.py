"""HIP path vs the CPU oracle on the same seeded inputs, through the C ABI (needs an MI355X).

Small cases span several tiles, ragged tails, mixed lengths and the degenerate cases of the method
(everything Initial, no candidates, k >= n_cand, k = 0, L = 1, zero-length windows, exact ties).
The full-size cases run the five benchmark workloads in the launch configuration bench.py times.
"""
from __future__ import annotations

import math
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
from parity import B, Case, check_selection, close_rel  # noqa: E402

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def cfg_of(Hq, Hkv, I, W, k, rep="quest", mode="separate", rep_num=1, kv="fp16"):
    return kvs.Config(num_q_heads=Hq, num_kv_heads=Hkv, initial_len=I, local_len=W, topk=k,
                      rep_method=rep, rep_num=rep_num, head_select_mode=mode, kv_type=kv)


def build_all_reps(case):
    c = case.cfg
    rp = ops.alloc_rep_pool(c, case.k_pool.shape[0], DEV)
    ids = []
    for i, L in enumerate(case.lens):
        ids.extend(int(x) for x in case.table[i, : L // B])
    if ids:
        ops.build_reps(c, case.k_pool, torch.tensor(ids, dtype=torch.int32), rp)
    case.built_ids = ids
    return rp


def run_full_check(case, label):
    """reps -> scores -> top-k -> attention (oracle selection) -> fused step (own selection)."""
    c, pb = case.cfg, case.pb
    say(f"[case] {label}: lens={case.lens[:6]}{'...' if len(case.lens) > 6 else ''} "
        f"Hq/Hkv={c.num_q_heads}/{c.num_kv_heads} I={c.initial_len} W={c.local_len} k={c.topk} "
        f"rep={c.rep_method}/{c.rep_num} mode={c.head_select_mode} kv={c.kv_type}")
    rp = build_all_reps(case)
    scores = ops.score_blocks(c, pb.q, rp, pb.block_table, pb.seq_lens)
    sel, cnt = ops.topk_blocks(c, scores, pb.seq_lens)
    refs = [case.oracle(i) for i in range(len(case.lens))]
    # oracle selection fed to the standalone attention
    G = c.groups
    osel = torch.full((len(case.lens), G, max(c.topk, 1)), -1, dtype=torch.int32)
    ocnt = torch.zeros((len(case.lens), G), dtype=torch.int32)
    for i, r in enumerate(refs):
        for gi in range(G):
            osel[i, gi, : len(r["sel"][gi])] = torch.tensor(r["sel"][gi], dtype=torch.int32)
            ocnt[i, gi] = len(r["sel"][gi])
    out_a = ops.sparse_decode_attn(c, pb.q, case.k_pool, case.v_pool, pb.block_table, pb.seq_lens,
                                   osel[:, :, : c.topk].to(DEV), ocnt.to(DEV))
    out_s, sel_s, cnt_s = ops.decode_step(c, pb.q, case.k_pool, case.v_pool, rp, pb.block_table,
                                          pb.seq_lens)
    torch.cuda.synchronize()
    kinds, errs = [], []
    for i, r in enumerate(refs):
        case.check_reps(rp, i, r)
        case.check_scores(scores, i, r)
        kinds += case.check_sel(sel, cnt, i, r)
        errs.append(case.check_out(out_a, i, r["out"], "attn(oracle sel)"))
        # fused step: its own selection, then attention over exactly that selection
        case.check_sel(sel_s, cnt_s, i, r)
        gsel = [[int(x) for x in sel_s[i, gi, : int(cnt_s[i, gi])].cpu()] for gi in range(G)]
        errs.append(case.check_out(out_s, i, case.oracle_attention(i, gsel), "decode_step"))
    assert torch.equal(sel, sel_s) and torch.equal(cnt, cnt_s)
    say(f"[ok] {label}: max err {max(errs):.2e}, selections {sorted(set(kinds))}")
    built = torch.tensor(case.built_ids, dtype=torch.long, device=DEV)
    return dict(rp=rp[built], scores=scores, sel=sel, cnt=cnt, out=out_s)


SMALL = [
    # (Hq, Hkv, I, W, k, rep, mode, rep_num, lens)
    (8, 8, 128, 1024, 8, "quest", "separate", 1, [8192]),
    (32, 8, 128, 512, 12, "max", "shared", 1, [5000, 129, 1, 7777]),
    (32, 8, 100, 300, 5, "mean", "shared", 1, [4000, 3001]),
    (64, 8, 128, 1000, 16, "quest", "separate", 1, [9000]),
    (16, 16, 0, 0, 7, "fix", "separate", 8, [3000, 2048]),
    (8, 2, 256, 640, 3, "quest", "shared", 1, [6000, 300, 1500]),
    (4, 1, 128, 200, 40, "mean", "separate", 1, [4000]),         # k >= n_cand
    (32, 8, 4096, 4096, 9, "quest", "separate", 1, [2000, 4096]),  # everything Initial
    (32, 8, 128, 4096, 0, "max", "shared", 1, [6000]),            # k = 0
    (16, 4, 1, 1, 6, "fix", "shared", 4, [2900, 128, 127]),
    (8, 4, 0, 130, 4, "fix", "separate", 128, [2000]),           # Fix with every token a rep
    (16, 2, 128, 2048, 24, "mean", "shared", 1, [290000]),       # long rows (> 2048 blocks)
    (16, 1, 128, 1024, 20, "quest", "separate", 1, [280000]),    # long rows, g = 16
    (8, 8, 128, 1024, 8000, "quest", "separate", 1, [8192, 300]),  # topk past the one-wave merge's LDS
    # long SEPARATE rows: selection from the 64-block chunks' summaries in the scoring launch
    (32, 8, 128, 4096, 64, "quest", "separate", 1, [2200 * 128 + 77, 3000 * 128, 2100 * 128 + 1]),
    (8, 4, 100, 900, 33, "max", "separate", 1, [4500 * 128 + 3]),
    (16, 16, 0, 0, 130, "fix", "separate", 8, [2049 * 128, 2600 * 128]),  # chunk 0 holds candidates
    (8, 8, 128, 2048 * 128, 64, "quest", "separate", 1, [2100 * 128 + 9]),  # k >= candidates
]


# Q8_0 caches: the same path over int8 codes and fp16 scales (kv_type), short and long rows
SMALL_Q8 = [
    (32, 8, 128, 512, 12, "quest", "separate", 1, [5000, 129, 1, 7777]),
    (32, 8, 100, 300, 5, "max", "shared", 1, [4000, 3001]),
    (16, 16, 0, 0, 7, "fix", "separate", 8, [3000, 2048]),
    (4, 1, 128, 200, 40, "mean", "separate", 1, [4000]),
    (16, 2, 128, 2048, 24, "mean", "shared", 1, [290000]),
    (32, 8, 128, 1024, 20, "quest", "separate", 1, [280000]),
]


SMALL_Q4 = [
    (32, 8, 128, 512, 12, "quest", "separate", 1, [5000, 129, 1, 7777]),
    (32, 8, 100, 300, 5, "max", "shared", 1, [4000, 3001]),
    (16, 2, 128, 2048, 24, "mean", "shared", 1, [290000]),
]


# INT8 caches with one fp32 scale per token and KV head
SMALL_I8 = [
    (32, 8, 128, 512, 12, "quest", "separate", 1, [5000, 129, 1, 7777]),
    (32, 8, 100, 300, 5, "max", "shared", 1, [4000, 3001]),
    (16, 16, 0, 0, 7, "fix", "separate", 8, [3000, 2048]),
    (16, 2, 128, 2048, 24, "mean", "shared", 1, [290000]),
]


@pytest.mark.parametrize("idx", range(len(SMALL_I8)),
                         ids=[f"i8-{s[5]}-{s[6]}-{s[0]}x{s[1]}-k{s[4]}" for s in SMALL_I8])
def test_small_cases_int8_pth(idx):
    Hq, Hkv, I, W, k, rep, mode, rn, lens = SMALL_I8[idx]
    c = cfg_of(Hq, Hkv, I, W, k, rep, mode, rn, kv="int8_pth")
    case = Case(c, lens, seed=kvsynth.mix_seed(79, idx), n_hot=3)
    run_full_check(case, f"small int8_pth {rep}/{mode} {Hq}x{Hkv}")


# INT4 caches with one fp32 scale and one zero point per token and KV head (includes a long SEPARATE
# row through the chunk summaries)
SMALL_I4 = [
    (32, 8, 128, 512, 12, "quest", "separate", 1, [5000, 129, 1, 7777]),
    (32, 8, 100, 300, 5, "max", "shared", 1, [4000, 3001]),
    (16, 16, 0, 0, 7, "fix", "separate", 8, [3000, 2048]),
    (16, 2, 128, 2048, 24, "mean", "shared", 1, [290000]),
    (16, 4, 128, 1024, 40, "quest", "separate", 1, [2300 * 128 + 11]),
]


@pytest.mark.parametrize("idx", range(len(SMALL_I4)),
                         ids=[f"i4-{s[5]}-{s[6]}-{s[0]}x{s[1]}-k{s[4]}" for s in SMALL_I4])
def test_small_cases_int4_pth(idx):
    Hq, Hkv, I, W, k, rep, mode, rn, lens = SMALL_I4[idx]
    c = cfg_of(Hq, Hkv, I, W, k, rep, mode, rn, kv="int4_pth")
    case = Case(c, lens, seed=kvsynth.mix_seed(80, idx), n_hot=3)
    run_full_check(case, f"small int4_pth {rep}/{mode} {Hq}x{Hkv}")


@pytest.mark.parametrize("idx", range(len(SMALL_Q4)),
                         ids=[f"q4-{s[5]}-{s[6]}-{s[0]}x{s[1]}-k{s[4]}" for s in SMALL_Q4])
def test_small_cases_q4(idx):
    Hq, Hkv, I, W, k, rep, mode, rn, lens = SMALL_Q4[idx]
    c = cfg_of(Hq, Hkv, I, W, k, rep, mode, rn, kv="q4_0")
    case = Case(c, lens, seed=kvsynth.mix_seed(78, idx), n_hot=3)
    run_full_check(case, f"small q4 {rep}/{mode} {Hq}x{Hkv}")


@pytest.mark.parametrize("idx", range(len(SMALL_Q8)),
                         ids=[f"q8-{s[5]}-{s[6]}-{s[0]}x{s[1]}-k{s[4]}" for s in SMALL_Q8])
def test_small_cases_q8(idx):
    Hq, Hkv, I, W, k, rep, mode, rn, lens = SMALL_Q8[idx]
    c = cfg_of(Hq, Hkv, I, W, k, rep, mode, rn, kv="q8_0")
    case = Case(c, lens, seed=kvsynth.mix_seed(77, idx), n_hot=3)
    run_full_check(case, f"small q8 {rep}/{mode} {Hq}x{Hkv}")


@pytest.mark.parametrize("idx", range(len(SMALL)),
                         ids=[f"{s[5]}-{s[6]}-{s[0]}x{s[1]}-k{s[4]}" for s in SMALL])
def test_small_cases(idx):
    Hq, Hkv, I, W, k, rep, mode, rn, lens = SMALL[idx]
    c = cfg_of(Hq, Hkv, I, W, k, rep, mode, rn)
    case = Case(c, lens, seed=kvsynth.mix_seed(7, idx), n_hot=3)
    run_full_check(case, f"small {rep}/{mode} {Hq}x{Hkv}")


def test_batch_odd_counts():
    """A batch of four 9K-33K sequences (over a thousand attended tiles in one call) with an odd k,
    odd Initial/Local counts and a partial last block."""
    c = cfg_of(32, 8, 128, 4096, 31, "quest", "separate")
    case = Case(c, [32768, 20000, 9000, 30001], seed=kvsynth.mix_seed(7, 99), n_hot=4)
    run_full_check(case, "batch of 4, odd counts")


def test_workspace_reused_across_calls():
    """One zero-filled workspace serves consecutive decode steps of different configs and batch
    sizes (its hand-off counters return to zero after every call): results equal those of fresh
    workspaces, bitwise."""
    cs = [cfg_of(32, 8, 128, 1024, 12, "max", "shared"), cfg_of(32, 8, 128, 1024, 9, "quest", "separate")]
    cases = [Case(cs[0], [20000, 7000, 15000], seed=61, n_hot=3), Case(cs[1], [9000], seed=62, n_hot=3)]
    reps = [build_all_reps(c) for c in cases]
    size = max(kvs.kvs_decode_step_workspace_size(c.cfg, len(c.lens), c.pb.max_blocks) for c in cases)
    ws = torch.zeros(size, dtype=torch.uint8, device=DEV)
    for rnd in range(2):
        for case, rp in zip(cases, reps):
            pb, c = case.pb, case.cfg
            fresh = ops.decode_step(c, pb.q, pb.k_pool, pb.v_pool, rp, pb.block_table, pb.seq_lens)
            reused = ops.decode_step(c, pb.q, pb.k_pool, pb.v_pool, rp, pb.block_table, pb.seq_lens, ws=ws)
            torch.cuda.synchronize()
            for a, b in zip(fresh, reused):
                assert torch.equal(a, b), (rnd, c.head_select_mode)
    assert int(ws[:65536].count_nonzero()) == 0, "counters not back to zero"


def test_exact_ties_take_lower_index():
    """Eleven identical blocks planted far above the rest (bitwise-equal scores); k = 5 cuts the tie
    group, so exactly its five lowest ids must be chosen, as the oracle does."""
    c = cfg_of(32, 8, 128, 512, 5, "quest", "separate")
    L = 64 * B
    s = kvsynth.make_sequence(11, L, 32, 8, 128, B, device=DEV)
    u = kvsynth.query_directions(s.q, 8).to(DEV)
    base = (s.K[10 * B:11 * B].float() + 6.0 * u[None]).half()
    for b in range(10, 21):
        s.K[b * B:(b + 1) * B] = base
    r = orc.decode_step(s.q.cpu().numpy(), s.K.cpu().numpy(), s.V.cpu().numpy(), B=B,
                        initial_len=128, local_len=512, topk=5, method="quest")
    assert all(x == [10, 11, 12, 13, 14] for x in r["sel"]), r["sel"]
    pb = kvsynth.page_batch([s], B, shuffle_seed=5, device=DEV)
    rp = ops.alloc_rep_pool(c, pb.k_pool.shape[0], DEV)
    ops.build_reps(c, pb.k_pool, pb.block_table[0, : L // B].cpu(), rp)
    scores = ops.score_blocks(c, pb.q, rp, pb.block_table, pb.seq_lens)
    sel, cnt = ops.topk_blocks(c, scores, pb.seq_lens)
    torch.cuda.synchronize()
    for h in range(8):
        grp = scores[0, h, 10:21]
        assert torch.all(grp == grp[0]), f"tie group not bitwise equal for head {h}"
        assert sel[0, h].tolist() == [10, 11, 12, 13, 14], (h, sel[0, h].tolist())


def test_exact_ties_long_row():
    """A SEPARATE row of 2,200 blocks (selected through the 64-block chunks' summaries) with eleven
    identical blocks 58..68 planted far above the rest: the tie group spans two chunks and k = 5 cuts
    it, so exactly blocks 58..62 must be chosen, as the oracle does."""
    c = cfg_of(32, 8, 128, 512, 5, "quest", "separate")
    L = 2200 * B
    say(f"[case] exact ties across a chunk boundary L={L} k=5")
    s = kvsynth.make_sequence(12, L, 32, 8, 128, B, device=DEV)
    u = kvsynth.query_directions(s.q, 8).to(DEV)
    base = (s.K[58 * B:59 * B].float() + 6.0 * u[None]).half()
    for b in range(58, 69):
        s.K[b * B:(b + 1) * B] = base
    r = orc.decode_step(s.q.cpu().numpy(), s.K.cpu().numpy(), s.V.cpu().numpy(), B=B,
                        initial_len=128, local_len=512, topk=5, method="quest")
    assert all(x == [58, 59, 60, 61, 62] for x in r["sel"]), r["sel"]
    pb = kvsynth.page_batch([s], B, shuffle_seed=6, device=DEV)
    rp = ops.alloc_rep_pool(c, pb.k_pool.shape[0], DEV)
    ops.build_reps(c, pb.k_pool, pb.block_table[0, : L // B].cpu(), rp)
    out, sel, cnt = ops.decode_step(c, pb.q, pb.k_pool, pb.v_pool, rp, pb.block_table, pb.seq_lens)
    torch.cuda.synchronize()
    for h in range(8):
        assert int(cnt[0, h]) == 5 and sel[0, h].tolist() == [58, 59, 60, 61, 62], (h, sel[0, h].tolist())
    say("[ok] exact ties across a chunk boundary")


@pytest.mark.parametrize("mode", ["hot", "flat"])
def test_long_row_chunk_overflow(mode):
    """A long SEPARATE row whose selection piles into one 64-block chunk (hot: 30 planted blocks inside
    blocks 128..191 with k = 20; flat: every key of that chunk shifted far above the rest with k = 40),
    so the chunk summaries cannot hold it and the selection falls back to the whole row: the result
    still equals the oracle's."""
    c = cfg_of(16, 4, 128, 1024, 20 if mode == "hot" else 40, "quest", "separate")
    L = 2300 * B + 11
    say(f"[case] long-row chunk overflow ({mode}) L={L} k={c.topk}")
    s = kvsynth.make_sequence(kvsynth.mix_seed(95, mode == "hot"), L, 16, 4, 128, B,
                              hot_range=(128, 192), n_hot=30 if mode == "hot" else 0, device=DEV)
    if mode == "flat":
        u = kvsynth.query_directions(s.q, 4).to(DEV)
        s.K[128 * B:192 * B] = (s.K[128 * B:192 * B].float() + 3.0 * u[None]).half()
    pb = kvsynth.page_batch([s], B, shuffle_seed=19, device=DEV)
    rp = ops.alloc_rep_pool(c, pb.k_pool.shape[0], DEV)
    ops.build_reps(c, pb.k_pool, pb.block_table[0, : L // B].cpu(), rp)
    out, sel, cnt = ops.decode_step(c, pb.q, pb.k_pool, pb.v_pool, rp, pb.block_table, pb.seq_lens)
    torch.cuda.synchronize()
    r = orc.decode_step(s.q.cpu().numpy(), s.K.cpu().numpy(), s.V.cpu().numpy(), B=B,
                        initial_len=128, local_len=1024, topk=c.topk, method="quest")
    in_chunk = 0
    for h in range(4):
        check_selection(sel[0, h].cpu().numpy(), cnt[0, h].item(), r["scores"][h], r["cand"], c.topk,
                        f"overflow sel h{h}")
        in_chunk = max(in_chunk, sum(1 for b in r["sel"][h] if 128 <= b < 192))
    assert in_chunk > 8, f"the case does not overflow a chunk summary ({in_chunk} in the chunk)"
    gsel = [[int(x) for x in sel[0, h, : int(cnt[0, h])].cpu()] for h in range(4)]
    toks = [orc.attended_tokens(L, B, r["init_end"], r["local_start"], gsel[j // 4]) for j in range(16)]
    ref = orc.attention(s.q.cpu().numpy(), s.K.cpu().numpy(), s.V.cpu().numpy(), toks)
    err = np.abs(out[0].double().cpu().numpy() - ref).max()
    say(f"[ok] long-row chunk overflow ({mode}): {in_chunk} selected blocks in one chunk, max err {err:.2e}")
    assert err <= 2e-3


def test_deterministic_and_split_invariant():
    """Two runs give bitwise-equal reps, scores, selections and outputs."""
    c = cfg_of(32, 8, 128, 1024, 16, "quest", "separate")
    case = Case(c, [20000, 7000], seed=21, n_hot=4)
    a = run_full_check(case, "determinism run 1")
    b = run_full_check(case, "determinism run 2")
    for key in ("rp", "scores", "sel", "cnt", "out"):
        assert torch.equal(a[key], b[key]), key


def test_shared_equals_sum_of_separate():
    cs = cfg_of(32, 8, 128, 1024, 10, "max", "separate")
    ch = cfg_of(32, 8, 128, 1024, 10, "max", "shared")
    case = Case(cs, [12000], seed=31, n_hot=2)
    rp = build_all_reps(case)
    pb = case.pb
    s_sep = ops.score_blocks(cs, pb.q, rp, pb.block_table, pb.seq_lens)
    s_sh = ops.score_blocks(ch, pb.q, rp, pb.block_table, pb.seq_lens)
    torch.cuda.synchronize()
    ie, ls, cand = orc.regions(12000, B, 128, 1024)
    tot = s_sep[0][:, cand].double().sum(0).cpu().numpy()
    got = s_sh[0, 0, cand].double().cpu().numpy()
    close_rel(got, tot, np.abs(tot).max(), "SHARED vs sum of SEPARATE")


def test_selection_reuse():
    """A selection made at length L stays valid at L + 300 (Local only grows): attention with the
    old selection matches the oracle over the same blocks."""
    c = cfg_of(32, 8, 128, 1024, 12, "quest", "separate")
    L0, L1 = 10000, 10300
    case = Case(c, [L1], seed=41, n_hot=3)
    pb = case.pb
    rp = build_all_reps(case)
    lens0 = torch.tensor([L0], dtype=torch.int32, device=DEV)
    _, sel0, cnt0 = ops.decode_step(c, pb.q, pb.k_pool, pb.v_pool, rp, pb.block_table, lens0)
    out1 = ops.sparse_decode_attn(c, pb.q, pb.k_pool, pb.v_pool, pb.block_table, pb.seq_lens,
                                  sel0, cnt0)
    torch.cuda.synchronize()
    gsel = [[int(x) for x in sel0[0, h, : int(cnt0[0, h])].cpu()] for h in range(8)]
    _, ls1, cand1 = orc.regions(L1, B, 128, 1024)
    assert all(set(s) <= set(cand1) for s in gsel)
    case.check_out(out1, 0, case.oracle_attention(0, gsel), "reused selection")


# ------------------------------------------------------------------------------------------------
# Full-size workloads (the five benchmark configurations)
# ------------------------------------------------------------------------------------------------
def test_full_8k_mha_quest():
    c = cfg_of(8, 8, 128, 1024, 8, "quest", "separate")
    case = Case(c, [8192], seed=20260000, n_hot=4, hot_per_head=False, shuffle=False)
    r = run_full_check(case, "full 8K 8/8 Quest k8")
    ref = case.oracle(0)
    hot = set(case.seqs[0].hot[0])
    assert all(hot <= set(s) for s in ref["sel"])  # planted blocks recalled


def test_full_32k_gqa64():
    c = cfg_of(64, 8, 128, 4096, 32, "quest", "separate")
    case = Case(c, [32768], seed=20260001, n_hot=8, hot_per_head=True, shuffle=False)
    run_full_check(case, "full 32K 64/8 Quest k32")


@pytest.mark.parametrize("rep", ["max", "mean"])
def test_full_128k_shared(rep):
    c = cfg_of(32, 8, 128, 4096, 96, rep, "shared")
    ncand = 991
    case = Case(c, [131072], seed=20260002, n_hot=math.ceil(0.05 * ncand), shuffle=False)
    run_full_check(case, f"full 128K 32/8 {rep} SHARED k96")


def test_full_128k_shared_q8():
    c = cfg_of(32, 8, 128, 4096, 96, "max", "shared", kv="q8_0")
    case = Case(c, [131072], seed=20260012, n_hot=50, shuffle=False)
    run_full_check(case, "full 128K 32/8 max SHARED k96, Q8_0 cache")


def test_full_128k_shared_q4():
    c = cfg_of(32, 8, 128, 4096, 96, "max", "shared", kv="q4_0")
    case = Case(c, [131072], seed=20260012, n_hot=50, shuffle=False)
    run_full_check(case, "full 128K 32/8 max SHARED k96, Q4_0 cache")


def test_full_128k_shared_int8_pth():
    c = cfg_of(32, 8, 128, 4096, 96, "max", "shared", kv="int8_pth")
    case = Case(c, [131072], seed=20260012, n_hot=50, shuffle=False)
    run_full_check(case, "full 128K 32/8 max SHARED k96, INT8 per-token-head cache")


def test_full_128k_shared_int4_pth():
    c = cfg_of(32, 8, 128, 4096, 96, "max", "shared", kv="int4_pth")
    case = Case(c, [131072], seed=20260012, n_hot=50, shuffle=False)
    run_full_check(case, "full 128K 32/8 max SHARED k96, INT4 per-token-head cache")


def test_full_mixed_batch_fix():
    c = cfg_of(32, 8, 128, 2048, 32, "fix", "shared", rep_num=8)
    g = torch.Generator().manual_seed(20260004)
    lens = torch.randint(16384, 131072 + 1, (16,), generator=g).tolist()
    case = Case(c, lens, seed=20260004, n_hot=8, shuffle=True)
    run_full_check(case, "full 16 x U[16K,128K] Fix8 SHARED k32")


def test_full_1m_layer():
    """One 1M-token layer in pool layout (identity table): every candidate's reps and score, the
    selection, and the attention output against the oracle."""
    c = cfg_of(32, 8, 128, 4096, 64, "quest", "separate")
    L = 1 << 20
    lo, hi = 1, (L - 4096) // B
    say(f"[case] full 1M layer: generating")
    q, kp, vp, hot = kvsynth.pool_layer(kvsynth.mix_seed(20260003, 0), L, 32, 8, hot_range=(lo, hi),
                                        n_hot=16, hot_per_head=True, device=DEV)
    nb = L // B
    table = torch.arange(nb, dtype=torch.int32, device=DEV)[None]
    lens = torch.tensor([L], dtype=torch.int32, device=DEV)
    rp = ops.alloc_rep_pool(c, nb, DEV)
    ops.build_reps(c, kp, torch.arange(nb, dtype=torch.int32), rp)
    out, sel, cnt = ops.decode_step(c, q[None], kp, vp, rp, table, lens)
    torch.cuda.synchronize()
    say("[case] full 1M layer: oracle")
    K = kvsynth.logical_from_pool(kp, table[0].cpu(), L).cpu().numpy()
    V = kvsynth.logical_from_pool(vp, table[0].cpu(), L).cpu().numpy()
    qn = q.cpu().numpy()
    r = orc.decode_step(qn, K, V, B=B, initial_len=128, local_len=4096, topk=64, method="quest")
    got_reps = rp[r["cand"]].double().cpu().numpy()
    assert np.array_equal(got_reps, r["reps"])
    scores = ops.score_blocks(c, q[None], rp, table, lens)
    torch.cuda.synchronize()
    for h in range(8):
        row = r["scores"][h]
        close_rel(scores[0, h, r["cand"]].double().cpu().numpy(), row, np.abs(row).max(),
                  f"1M scores h{h}")
        check_selection(sel[0, h].cpu().numpy(), cnt[0, h].item(), row, r["cand"], 64,
                        f"1M sel h{h}")
    # planted-block recall is a property of the synthetic data, not of parity: report it
    recall = np.mean([len(set(hot[h]) & set(sel[0, h].tolist())) / len(hot[h]) for h in range(8)])
    say(f"[info] 1M planted-block recall {recall:.3f}")
    gsel = [[int(x) for x in sel[0, h, : int(cnt[0, h])].cpu()] for h in range(8)]
    toks = [orc.attended_tokens(L, B, r["init_end"], r["local_start"], gsel[j // 4]) for j in range(32)]
    ref = orc.attention(qn, K, V, toks)
    err = np.abs(out[0].double().cpu().numpy() - ref).max()
    say(f"[ok] full 1M layer: max err {err:.2e}")
    assert err <= 2e-3
