"""Brute force on tiny hand-built caches, written independently of the oracle.

Exact rational arithmetic (Fraction) for reps, scores and group sums; token-by-token region
classification by loops; top-k by counting, for each candidate, the candidates that beat it
(score greater, or equal with a lower block index) -- a different algorithm from the oracle's sort.
Attention uses a per-token float loop with math.fsum.  Inputs are small dyadic numbers drawn from a
coarse grid, so ties are frequent.
"""
from __future__ import annotations

import math
import random
from fractions import Fraction

import numpy as np

from oracle import kvs_oracle as orc

METHODS = ("quest", "max", "mean", "fix")


def bf_regions(L, B, I, W):
    init_end = 0
    while init_end < I:
        init_end += B
    if L <= init_end:
        return L, L, []
    loc = 0
    while loc + B <= L - W:
        loc += B
    loc = max(loc, init_end)
    cand = []
    b = init_end // B
    while (b + 1) * B <= loc:
        cand.append(b)
        b += 1
    return init_end, loc, cand


def bf_reps(K, B, b, h, method, rep_num):
    rows = [[Fraction(K[t][h][c]) for c in range(len(K[0][0]))] for t in range(b * B, (b + 1) * B)]
    d = len(rows[0])
    if method == "quest":
        return [[min(r[c] for r in rows) for c in range(d)], [max(r[c] for r in rows) for c in range(d)]]
    if method == "max":
        return [[max(r[c] for r in rows) for c in range(d)]]
    if method == "mean":
        return [[sum(r[c] for r in rows) / B for c in range(d)]]
    stride = B // rep_num
    return [rows[r * stride] for r in range(rep_num)]


def bf_head_score(qj, reps, method):
    if method == "quest":
        kmin, kmax = reps
        return sum(max(qc * a, qc * b) for qc, a, b in zip(qj, kmax, kmin))
    return sum(sum(qc * x for qc, x in zip(qj, rep)) for rep in reps)


def bf_decode(q, K, V, B, I, W, k, method, rep_num, mode):
    L, Hkv, d = len(K), len(K[0]), len(K[0][0])
    Hq = len(q)
    g = Hq // Hkv
    qf = [[Fraction(x) for x in row] for row in q]
    ie, ls, cand = bf_regions(L, B, I, W)
    head = {}
    reps = {}
    for b in cand:
        for h in range(Hkv):
            reps[(b, h)] = bf_reps(K, B, b, h, method, rep_num)
        for j in range(Hq):
            head[(b, j)] = bf_head_score(qf[j], reps[(b, j // g)], method)
    groups = list(range(Hkv)) if mode == "separate" else [0]
    score = {}
    for gi in groups:
        for b in cand:
            js = [j for j in range(Hq) if (j // g == gi or mode == "shared")]
            score[(gi, b)] = sum(head[(b, j)] for j in js)
    sel = {}
    for gi in groups:
        chosen = []
        for b in cand:
            beaten_by = sum(1 for c in cand if score[(gi, c)] > score[(gi, b)]
                            or (score[(gi, c)] == score[(gi, b)] and c < b))
            if beaten_by < k:
                chosen.append(b)
        sel[gi] = chosen
    out = []
    for j in range(Hq):
        h = j // g
        gi = h if mode == "separate" else 0
        T = [t for t in range(L) if t < ie or t >= ls or (t // B in sel[gi])]
        z = [sum(float(q[j][c]) * float(K[t][h][c]) for c in range(d)) / math.sqrt(d) for t in T]
        m = max(z)
        w = [math.exp(x - m) for x in z]
        den = math.fsum(w)
        out.append([math.fsum(wi * float(V[t][h][c]) for wi, t in zip(w, T)) / den for c in range(d)])
    return dict(cand=cand, reps=reps, head=head, score=score, sel=sel, out=out, ie=ie, ls=ls)


def _grid(rng, shape):
    # values in {-2, -1.75, ..., 2}: exact in fp16, frequent ties
    return (rng.integers(-8, 9, size=shape) / 4.0).astype(np.float64)


def _cases(n=60, seed=1234):
    rng = np.random.default_rng(seed)
    pyr = random.Random(seed)
    for i in range(n):
        B = pyr.choice([2, 3, 4])
        d = pyr.choice([2, 4])
        Hkv = pyr.choice([1, 2])
        Hq = Hkv * pyr.choice([1, 2])
        L = pyr.randint(1, 40)
        I = pyr.randint(0, 9)
        W = pyr.randint(0, 12)
        k = pyr.randint(0, 6)
        method = METHODS[i % 4]
        rep_num = pyr.choice([r for r in (1, 2, 3, 4) if B % r == 0]) if method == "fix" else 1
        mode = "separate" if (i // 4) % 2 == 0 else "shared"
        K = _grid(rng, (L, Hkv, d))
        if L >= 3 * B and i % 3 == 0:       # plant exact ties: copy a block onto the next one
            K[B:2 * B] = K[2 * B:3 * B]
        V = _grid(rng, (L, Hkv, d))
        q = _grid(rng, (Hq, d))
        yield dict(B=B, d=d, Hkv=Hkv, Hq=Hq, L=L, I=I, W=W, k=k, method=method, rep_num=rep_num,
                   mode=mode, K=K, V=V, q=q)


def check_against_bruteforce(o=orc, n=60):
    for c in _cases(n):
        bf = bf_decode(c["q"].tolist(), c["K"].tolist(), c["V"].tolist(), c["B"], c["I"], c["W"],
                       c["k"], c["method"], c["rep_num"], c["mode"])
        r = o.decode_step(c["q"], c["K"], c["V"], B=c["B"], initial_len=c["I"], local_len=c["W"],
                          topk=c["k"], method=c["method"], rep_num=c["rep_num"], mode=c["mode"])
        tag = {k: v for k, v in c.items() if k not in ("K", "V", "q")}
        assert (r["init_end"], r["local_start"], r["cand"]) == (bf["ie"], bf["ls"], bf["cand"]), tag
        for bi, b in enumerate(r["cand"]):
            for h in range(c["Hkv"]):
                want = [[float(x) for x in rep] for rep in bf["reps"][(b, h)]]
                got = r["reps"][bi, h].tolist()
                if c["method"] == "mean" and c["B"] == 3:
                    assert np.allclose(got, want, rtol=1e-15, atol=1e-15), tag
                else:
                    assert got == want, tag
            for j in range(c["Hq"]):
                assert abs(r["head_scores"][bi, j] - float(bf["head"][(b, j)])) <= 1e-12, tag
        for gi, sel in bf["sel"].items():
            for bi, b in enumerate(r["cand"]):
                assert abs(r["scores"][gi, bi] - float(bf["score"][(gi, b)])) <= 1e-12, tag
            assert r["sel"][gi] == sel, (tag, r["sel"][gi], sel)
        assert np.allclose(r["out"], np.asarray(bf["out"]), rtol=0, atol=1e-12), tag


def test_oracle_matches_bruteforce():
    check_against_bruteforce(orc, n=200)


def test_bruteforce_covers_edge_cases():
    """The generated cases include: no candidates (L <= I_b), k >= n_cand, k = 0, ties, both modes."""
    seen = set()
    for c in _cases(200):
        ie, ls, cand = bf_regions(c["L"], c["B"], c["I"], c["W"])
        if not cand:
            seen.add("no_cand")
        elif c["k"] >= len(cand):
            seen.add("k_ge_ncand")
        elif c["k"] == 0:
            seen.add("k0")
        if c["L"] <= ie:
            seen.add("all_initial")
        if c["L"] % c["B"]:
            seen.add("ragged")
        seen.add(c["mode"])
    assert {"no_cand", "k_ge_ncand", "k0", "all_initial", "ragged", "separate", "shared"} <= seen
