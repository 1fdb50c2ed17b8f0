"""Dynamic reps on the GPU against the oracle (needs an MI355X).

Token importance (the attention the last n_obs queries pay each cached token, summed over the
group's query heads, causal; over a quantized cache the keys are its cached values) is compared
within 1e-4 relative to the row scale; the rep tokens a
block picks must be the oracle's, or differ only inside the tie band of the rep_num-th score; the
decode step with Dynamic reps is then held to the usual rules, given the reps the GPU built.
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
from parity import ATOL_OUT, B, REL, Case, check_selection, close_rel  # noqa: E402

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dyn_cfg(Hq, Hkv, mode, rep_num, I=128, W=512, k=8, kv="fp16"):
    return kvs.Config(num_q_heads=Hq, num_kv_heads=Hkv, initial_len=I, local_len=W, topk=k,
                      rep_method="dynamic", rep_num=rep_num, head_select_mode=mode, kv_type=kv)


def run_importance(case, n_obs, seed):
    c, pb = case.cfg, case.pb
    q_obs = kvsynth.randn_fp16((len(case.lens), n_obs, c.num_q_heads, 128), seed, DEV)
    imp = ops.token_importance(c, q_obs, case.k_pool, pb.block_table, pb.seq_lens)
    torch.cuda.synchronize()
    refs = [orc.token_importance(q_obs[i].cpu().numpy(), case.host[i][1], c.head_select_mode)
            for i in range(len(case.lens))]
    got = imp.double().cpu().numpy()
    for i, (L, ref) in enumerate(zip(case.lens, refs)):
        close_rel(got[i, :, :L], ref, np.abs(ref).max(axis=-1, keepdims=True), f"importance seq {i}")
        assert np.all(got[i, :, L:] == 0.0), f"importance past L, seq {i}"
    return imp, refs


IMP_CASES = [
    # (Hq, Hkv, mode, n_obs, lens, kv): over a quantized cache the keys are its cached values
    (8, 2, "separate", 5, [1000, 300], "fp16"),
    (32, 8, "shared", 32, [4000], "fp16"),
    (4, 4, "separate", 1, [129, 257], "fp16"),
    (16, 1, "shared", 40, [2000], "fp16"),
    (8, 8, "separate", 130, [700], "fp16"),
    (8, 2, "separate", 5, [1000, 300], "q8_0"),
    (32, 8, "shared", 32, [4000], "q4_0"),
    (16, 4, "separate", 8, [2000], "int8_pth"),
    (16, 4, "shared", 8, [2000], "int4_pth"),
]


@pytest.mark.parametrize("idx", range(len(IMP_CASES)))
def test_importance(idx):
    Hq, Hkv, mode, n_obs, lens, kv = IMP_CASES[idx]
    say(f"[case] importance {Hq}x{Hkv} {mode} n_obs={n_obs} lens={lens} kv={kv}")
    c = dyn_cfg(Hq, Hkv, mode, 2, kv=kv)
    case = Case(c, lens, seed=kvsynth.mix_seed(501, idx))
    run_importance(case, n_obs, kvsynth.mix_seed(502, idx))


def picked_tokens(rep_rows, block_rows):
    """Token offsets of the rep rows, found among the block's K rows (random rows are distinct)."""
    out = []
    for r in rep_rows:
        hit = np.nonzero(np.all(block_rows == r[None, :], axis=1))[0]
        assert len(hit) == 1, "a rep row is not one of the block's keys"
        out.append(int(hit[0]))
    return out


DYN_CASES = [
    # (Hq, Hkv, mode, rep_num, n_obs, k, lens, kv)
    (32, 8, "shared", 1, 16, 12, [6000, 3000], "fp16"),
    (8, 2, "separate", 4, 8, 6, [5000], "fp16"),
    (16, 4, "separate", 3, 4, 40, [1500], "fp16"),        # rep_num not dividing the block; k >= n_cand
    (16, 2, "shared", 2, 8, 24, [280000], "fp16"),        # long rows: the selection launch of > 2048 blocks
    (32, 8, "shared", 1, 16, 12, [6000, 3000], "q8_0"),   # quantized caches: reps are cached values
    (8, 2, "separate", 4, 8, 6, [5000], "q4_0"),
    (16, 4, "separate", 3, 4, 10, [4500], "int8_pth"),
    (16, 4, "separate", 3, 4, 10, [4500], "int4_pth"),
]


@pytest.mark.parametrize("idx", range(len(DYN_CASES)))
def test_dynamic_reps_and_step(idx):
    Hq, Hkv, mode, rn, n_obs, k, lens, kv = DYN_CASES[idx]
    say(f"[case] dynamic reps {Hq}x{Hkv} {mode} rep_num={rn} n_obs={n_obs} k={k} lens={lens} kv={kv}")
    c = dyn_cfg(Hq, Hkv, mode, rn, k=k, kv=kv)
    case = Case(c, lens, seed=kvsynth.mix_seed(503, idx), n_hot=3)
    pb = case.pb
    imp, imp_ref = run_importance(case, n_obs, kvsynth.mix_seed(504, idx))
    rp = ops.alloc_rep_pool(c, pb.k_pool.shape[0], DEV)
    rp.zero_()
    ops.build_dynamic_reps(c, case.k_pool, imp, pb.block_table, pb.seq_lens, rp)
    out, sel, cnt = ops.decode_step(c, pb.q, case.k_pool, case.v_pool, rp, pb.block_table, pb.seq_lens)
    scores = ops.score_blocks(c, pb.q, rp, pb.block_table, pb.seq_lens)
    torch.cuda.synchronize()
    G = c.groups
    bands = 0
    for i, L in enumerate(case.lens):
        q, K, V = case.host[i]
        init_end, local_start, cand = orc.regions(L, B, c.initial_len, c.local_len)
        phys = case.table[i, cand]
        gpu_reps = rp[torch.as_tensor(phys, dtype=torch.long, device=DEV)].double().cpu().numpy()
        ref_reps, ref_pick = orc.dynamic_reps(K, imp_ref[i], B, rn, mode, cand)
        for n, b in enumerate(cand):
            for h in range(Hkv):
                # the block's K rows as a rep stores them (fp16; the identity for an fp16 cache)
                rows = orc.stored_reps(np.asarray(K[b * B:(b + 1) * B, h, :], np.float64), "fix")
                got = picked_tokens(gpu_reps[n, h], rows)
                assert got == sorted(got), f"reps not in token order seq {i} block {b} head {h}"
                want = ref_pick[n, h].tolist()
                if got != want:  # only inside the tie band of the rep_num-th score
                    row = imp_ref[i][h if mode == "separate" else 0, b * B:(b + 1) * B]
                    kth = sorted(row, reverse=True)[rn - 1]
                    beta = REL * max(abs(kth), np.abs(row).max())
                    for t in set(got) ^ set(want):
                        assert abs(row[t] - kth) <= beta, (i, b, h, got, want)
                    bands += 1
        # the rest of the step, given the reps the GPU built
        ref = orc.decode_step(q, K, V, B=B, initial_len=c.initial_len, local_len=c.local_len, topk=k,
                              method="dynamic", rep_num=rn, mode=mode, reps=gpu_reps)
        got_s = scores[i].double().cpu().numpy()
        for gi in range(G):
            if cand:
                row = ref["scores"][gi]
                close_rel(got_s[gi, cand], row, np.abs(row).max(), f"dynamic scores seq {i} grp {gi}")
            check_selection(sel[i, gi].cpu().numpy(), cnt[i, gi].item(), ref["scores"][gi] if cand else [],
                            cand, k, f"dynamic sel seq {i} grp {gi}")
        gsel = [[int(x) for x in sel[i, gi, : int(cnt[i, gi])].cpu()] for gi in range(G)]
        g = c.num_q_heads // c.num_kv_heads
        toks = [orc.attended_tokens(L, B, init_end, local_start, gsel[(j // g) if mode == "separate" else 0])
                for j in range(c.num_q_heads)]
        want_out = orc.attention(q, K, V, toks)
        err = float(np.abs(out[i].double().cpu().numpy() - want_out).max())
        assert err <= ATOL_OUT, f"dynamic step out seq {i}: {err:.3e}"
    say(f"[ok] dynamic {idx}: rep picks in the tie band: {bands}")
