"""GPU-vs-oracle comparison rules and case runners for the parity tests.

Acceptance (same seeded inputs on both sides):
  * Quest / Max / Fix reps: equal values (fp16 min, max and copies are exact).
  * Mean reps and block scores: |gpu - ref| <= 1e-4 * max(|ref|, max|row|), row = one rep's 128
    channels or one (sequence, group)'s candidate scores.  Non-candidates must be -inf.
  * Selection: equal to the oracle's, unless the oracle's k-th and (k+1)-th scores are within
    1e-4 relative; then any k_eff-set that holds every block scoring clearly above the k-th and only
    blocks scoring at least the (k+1)-th (both within the band) is accepted.
  * Attention: max |gpu - ref| <= 2e-3, where ref is the oracle's attention over the GPU's own
    selection (a different legal selection attends different tokens).
  * A Q8_0, Q4_0, INT8 or INT4 (per token and head) cache (kv_type): the oracle works on the dequantized
    keys and values of its own
    quantization of the same fp16 rows (the codes are bit-exact, tests/test_gpu_q8.py) and on reps
    stored as the rep pool stores them (fp16, Mean fp32).  The same bounds hold: the kernels round
    each dequantized value to fp16 once (relative 2**-11 per element), which moves the outputs by
    about 1e-4 here.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import kvsynth
from oracle import kvs_oracle as orc

REL = 1e-4
ATOL_OUT = 2e-3
B = 128


def method_name(m):
    return {0: "quest", 1: "max", 2: "mean", 3: "fix"}.get(m, m)


def close_rel(got, ref, row_scale, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    tol = REL * np.maximum(np.abs(ref), row_scale)
    bad = np.abs(got - ref) > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} values off; worst |d|="
                           f"{np.abs(got - ref)[bad].max():.3e} at {np.argwhere(bad)[:3].tolist()}")


def check_selection(gpu_sel, gpu_cnt, ref_scores_row, cand, k, what):
    """gpu_sel: ascending logical ids (len >= k_eff, -1 padded); ref_scores_row aligned with cand."""
    k_eff = min(k, len(cand))
    assert int(gpu_cnt) == k_eff, f"{what}: count {int(gpu_cnt)} != {k_eff}"
    got = [int(x) for x in gpu_sel[:k_eff]]
    assert all(x == -1 for x in gpu_sel[k_eff:k]), f"{what}: padding"
    assert got == sorted(got) and len(set(got)) == k_eff, f"{what}: not ascending/distinct {got}"
    ref = orc.select_topk(ref_scores_row, cand, k)
    if got == ref:
        return "exact"
    assert 0 < k_eff < len(cand), f"{what}: differs without a tie band {got} vs {ref}"
    s = {b: float(v) for b, v in zip(cand, ref_scores_row)}
    ordered = sorted(cand, key=lambda b: (-s[b], b))
    sk, sk1 = s[ordered[k_eff - 1]], s[ordered[k_eff]]
    beta = REL * abs(sk)
    assert sk - sk1 < beta, f"{what}: selection differs with a clear gap {got} vs {ref}"
    for b in cand:
        if s[b] > sk + beta:
            assert b in got, f"{what}: block {b} clearly above the k-th is missing"
    for b in got:
        assert b in s and s[b] >= sk1 - beta, f"{what}: block {b} clearly below the (k+1)-th"
    return "tie-band"


class Case:
    """One batch on the GPU plus its host copy for the oracle."""

    def __init__(self, cfg, lens, seed, *, n_hot=0, hot_per_head=False, shuffle=True,
                 device="cuda", spare_blocks=3):
        self.cfg = cfg
        kv = getattr(cfg, "kv_type", "fp16")
        self.kv = {1: "q8_0", 2: "q4_0", 3: "int8_pth", 4: "int4_pth", 0: "fp16"}.get(kv, kv)
        self.q8 = self.kv != "fp16"  # a quantized cache (Q8_0, Q4_0, or INT8 / INT4 per token and head)
        seqs = []
        for i, L in enumerate(lens):
            ie, ls, cand = orc.regions(L, B, cfg.initial_len, cfg.local_len)
            lo, hi = (cand[0], cand[-1] + 1) if cand else (0, 0)
            seqs.append(kvsynth.make_sequence(kvsynth.mix_seed(seed, i), L, cfg.num_q_heads,
                                              cfg.num_kv_heads, 128, B, hot_range=(lo, hi),
                                              n_hot=n_hot, hot_per_head=hot_per_head,
                                              device=device))
        self.seqs = seqs
        self.pb = kvsynth.page_batch(seqs, B, shuffle_seed=seed if shuffle else None,
                                     spare_blocks=spare_blocks, device=device)
        self.host = [(s.q.cpu().numpy(), s.K.cpu().numpy(), s.V.cpu().numpy()) for s in seqs]
        self.table = self.pb.block_table.cpu().numpy()
        self.lens = list(lens)
        self.k_pool, self.v_pool = self.pb.k_pool, self.pb.v_pool
        if self.q8:  # the GPU pools quantized by the library, the host rows by the oracle
            from block_sparse_kv_amd import ops
            n_phys = self.pb.k_pool.shape[0]
            ids = torch.arange(n_phys, dtype=torch.int32)
            self.k_pool = ops.quantize_kv(cfg, self.pb.k_pool, ids, ops.alloc_q8_pool(cfg, n_phys, device))
            self.v_pool = ops.quantize_kv(cfg, self.pb.v_pool, ids, ops.alloc_q8_pool(cfg, n_phys, device))
            qf, df = {"q8_0": (orc.quantize_q8_0, orc.dequantize_q8_0),
                      "q4_0": (orc.quantize_q4_0, orc.dequantize_q4_0),
                      "int8_pth": (orc.quantize_int8_pth, orc.dequantize_int8_pth),
                      "int4_pth": (orc.quantize_int4_pth, orc.dequantize_int4_pth)}[self.kv]
            self.host = [(q, df(*qf(K)), df(*qf(V))) for q, K, V in self.host]

    # --- oracle side --------------------------------------------------------------------------
    def oracle(self, i):
        c = self.cfg
        q, K, V = self.host[i]
        m = method_name(c.rep_method)
        reps = None
        if self.q8:
            cand = orc.regions(K.shape[0], B, c.initial_len, c.local_len)[2]
            reps = orc.stored_reps(orc.block_reps(K, B, m, c.rep_num, blocks=cand), m)
        return orc.decode_step(q, K, V, B=B, initial_len=c.initial_len, local_len=c.local_len,
                               topk=c.topk, method=m, rep_num=c.rep_num,
                               mode=c.head_select_mode, scale=(c.softmax_scale or None), reps=reps)

    def oracle_attention(self, i, sel_per_group):
        c = self.cfg
        q, K, V = self.host[i]
        L = K.shape[0]
        ie, ls, _ = orc.regions(L, B, c.initial_len, c.local_len)
        g = c.num_q_heads // c.num_kv_heads
        toks = []
        for j in range(c.num_q_heads):
            gi = j // g if c.head_select_mode == "separate" else 0
            toks.append(orc.attended_tokens(L, B, ie, ls, sel_per_group[gi]))
        return orc.attention(q, K, V, toks, c.softmax_scale or None)

    # --- comparisons ----------------------------------------------------------------------------
    def check_reps(self, rep_pool, i, ref):
        """ref: oracle result of sequence i (reps of its candidates)."""
        c = self.cfg
        if not ref["cand"]:
            return
        ids = torch.as_tensor(self.table[i, ref["cand"]], dtype=torch.long, device=rep_pool.device)
        got = rep_pool.index_select(0, ids).double().cpu().numpy()  # [n][Hkv][R][d]
        want = ref["reps"]
        if method_name(c.rep_method) == "mean":
            row = np.abs(want).max(axis=-1, keepdims=True)
            close_rel(got, want, row, f"mean reps seq {i}")
        else:
            assert np.array_equal(got, want), f"reps seq {i}: {np.argwhere(got != want)[:3]}"

    def check_scores(self, scores, i, ref):
        G = scores.shape[1]
        got = scores[i].double().cpu().numpy()
        cand = ref["cand"]
        for gi in range(G):
            mask = np.ones(got.shape[1], dtype=bool)
            if cand:
                mask[cand] = False
                row = ref["scores"][gi]
                close_rel(got[gi, cand], row, np.abs(row).max(), f"scores seq {i} grp {gi}")
            assert np.all(np.isneginf(got[gi, mask])), f"non-candidate scores seq {i} grp {gi}"

    def check_sel(self, sel, cnt, i, ref):
        kinds = []
        for gi in range(sel.shape[1]):
            kinds.append(check_selection(sel[i, gi].cpu().numpy(), cnt[i, gi].item(),
                                         ref["scores"][gi] if ref["cand"] else [], ref["cand"],
                                         self.cfg.topk, f"sel seq {i} grp {gi}"))
        return kinds

    def check_out(self, out, i, ref_out, what="out"):
        got = out[i].double().cpu().numpy()
        err = np.abs(got - ref_out).max()
        assert np.isfinite(got).all(), f"{what} seq {i}: non-finite output"
        assert err <= ATOL_OUT, f"{what} seq {i}: max abs err {err:.3e}"
        return err
