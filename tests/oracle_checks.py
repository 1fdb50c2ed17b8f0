"""Checks that pin the CPU oracle to things other than itself.

Each ``check_*`` takes the oracle module (so the mutation tests can hand in a deliberately broken
copy) and raises AssertionError on failure.  What each one rests on:
  * exact integer arithmetic (every fp16 value is an integer multiple of 2**-24);
  * torch's scaled_dot_product_attention in float64 (a library routine sharing no code with the oracle);
  * closed forms and identities of the definitions (Mean linearity, Fix = rows of K, SHARED = sum
    of SEPARATE, softmax shift invariance, q = 0 gives the mean of V);
  * hand-worked cases in tests/golden/hand_worked.json, q8_0_worked.json, q4_0_worked.json and
    int8_pth_worked.json, int4_pth_worked.json;
  * the rounding bound, code range and block width of the Q8_0 format;
  * planted-block recall of the selection.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import kvsynth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def exact_int(x) -> list:
    """fp16-representable floats -> exact integers in units of 2**-24."""
    a = np.asarray(x, dtype=np.float64) * (1 << 24)
    assert np.all(a == np.round(a)), "input is not fp16-representable"
    return a.astype(np.int64)


def small_seq(seed, L=1000, Hq=4, Hkv=2, d=16, B=16, **kw):
    s = kvsynth.make_sequence(seed, L, Hq, Hkv, d, B, **kw)
    return s.q.numpy(), s.K.numpy(), s.V.numpy(), s


# ------------------------------------------------------------------------------------------ reps
def check_quest_upper_bound(orc, seeds=(1, 2, 3)):
    """Quest score >= max_t q.k_t for every block and head, in exact integers (2**-48 units)."""
    for seed in seeds:
        q, K, V, _ = small_seq(seed)
        L, Hkv, d = K.shape
        B = 16
        Hq = q.shape[0]
        g = Hq // Hkv
        blocks = list(range(L // B))
        reps = orc.block_reps(K, B, orc.QUEST, blocks=blocks)
        s = orc.head_scores(q, reps, orc.QUEST)
        qi = exact_int(q)
        Ki = exact_int(K)
        for bi, b in enumerate(blocks):
            for j in range(Hq):
                h = j // g
                dots = [int(np.dot(qi[j].astype(object), Ki[t, h].astype(object)))
                        for t in range(b * B, (b + 1) * B)]
                true_max = max(dots) / float(1 << 48)
                # fp64 rounding of a 16-term sum is far below 1e-9 here
                assert s[bi, j] >= true_max - 1e-9 * max(1.0, abs(true_max)), (seed, b, j)


def check_quest_tight_and_units(orc):
    """A block whose keys are all equal has Quest score == q.k exactly; a unit query e_c scores
    kmax_c and -e_c scores -kmin_c (pins channel indexing and which of min/max is which)."""
    rng = np.random.default_rng(7)
    B, d, Hkv, Hq = 8, 16, 2, 4
    g = Hq // Hkv
    K = np.round(rng.standard_normal((4 * B, Hkv, d)) * 64) / 64  # dyadic: exact everywhere
    K[B:2 * B] = K[B]                                              # block 1: one repeated row
    q = np.round(rng.standard_normal((Hq, d)) * 64) / 64
    reps = orc.block_reps(K, B, orc.QUEST)
    s = orc.head_scores(q, reps, orc.QUEST)
    for j in range(Hq):
        assert s[1, j] == float(np.dot(q[j], K[B, j // g])), j
    kmax = K.reshape(4, B, Hkv, d).max(axis=1)
    kmin = K.reshape(4, B, Hkv, d).min(axis=1)
    for c in range(d):
        e = np.zeros((Hkv, d))
        e[:, c] = 1.0
        se = orc.head_scores(e, reps, orc.QUEST)        # Hq = Hkv: head j reads KV head j
        assert np.array_equal(se[:, 0], kmax[:, 0, c]) and np.array_equal(se[:, 1], kmax[:, 1, c])
        sn = orc.head_scores(-e, reps, orc.QUEST)
        assert np.array_equal(sn[:, 0], -kmin[:, 0, c]) and np.array_equal(sn[:, 1], -kmin[:, 1, c])


def check_rep_closed_forms(orc, seed=11):
    """Mean score = (1/B) sum_t q.k_t (linearity); Quest >= Max-rep score and >= Mean score;
    kmin <= mean <= kmax; Quest >= every Fix rep's dot; Fix reps are K rows at r*B/rep_num."""
    q, K, V, _ = small_seq(seed, L=512, Hq=4, Hkv=2, d=16, B=16)
    B, Hq, Hkv = 16, 4, 2
    g = Hq // Hkv
    nb = K.shape[0] // B
    rq = orc.block_reps(K, B, orc.QUEST)
    rmax = orc.block_reps(K, B, orc.MAX)
    rmean = orc.block_reps(K, B, orc.MEAN)
    rfix = orc.block_reps(K, B, orc.FIX, rep_num=4)
    sq = orc.head_scores(q, rq, orc.QUEST)
    smax = orc.head_scores(q, rmax, orc.MAX)
    smean = orc.head_scores(q, rmean, orc.MEAN)
    K64 = K.astype(np.float64)
    q64 = q.astype(np.float64)
    for b in range(nb):
        for j in range(Hq):
            h = j // g
            direct = sum(float(np.dot(q64[j], K64[t, h])) for t in range(b * B, (b + 1) * B)) / B
            assert abs(smean[b, j] - direct) <= 1e-12 * max(1.0, abs(direct)), (b, j)
            assert sq[b, j] >= smax[b, j] - 1e-12 and sq[b, j] >= smean[b, j] - 1e-12
            for r in range(4):
                assert np.array_equal(rfix[b, h, r], K64[b * B + r * (B // 4), h])
                assert sq[b, j] >= float(np.dot(q64[j], rfix[b, h, r])) - 1e-12
        assert np.all(rq[b, :, 0] <= rmean[b, :, 0] + 1e-15)
        assert np.all(rmean[b, :, 0] <= rq[b, :, 1] + 1e-15)
        assert np.array_equal(rmax[b, :, 0], rq[b, :, 1])


def check_hand_worked(orc):
    gd = golden()
    c = gd["quest_block"]
    K = np.asarray(c["keys"], dtype=np.float64)[:, None, :]   # [B][Hkv=1][d]
    q = np.asarray([c["q"]])
    rq = orc.block_reps(K, c["B"], orc.QUEST)
    assert np.array_equal(rq[0, 0, 0], c["kmin"]) and np.array_equal(rq[0, 0, 1], c["kmax"])
    assert np.array_equal(orc.block_reps(K, c["B"], orc.MEAN)[0, 0, 0], c["mean"])
    assert orc.head_scores(q, rq, orc.QUEST)[0, 0] == c["quest_score"]
    assert orc.head_scores(q, orc.block_reps(K, 2, orc.MAX), orc.MAX)[0, 0] == c["max_score"]
    assert orc.head_scores(q, orc.block_reps(K, 2, orc.MEAN), orc.MEAN)[0, 0] == c["mean_score"]
    assert orc.head_scores(q, orc.block_reps(K, 2, orc.FIX, 1), orc.FIX)[0, 0] == c["fix1_score"]
    assert orc.head_scores(q, orc.block_reps(K, 2, orc.FIX, 2), orc.FIX)[0, 0] == c["fix2_score"]
    for key in ("decode_step", "tie"):
        c = gd[key]
        K = np.asarray(c["keys"], dtype=np.float64)[:, None, :]
        V = np.zeros_like(K)
        q = np.asarray(c["q"], dtype=np.float64)
        r = orc.decode_step(q, K, V, B=c["B"], initial_len=c["initial_len"],
                            local_len=c["local_len"], topk=c["topk"], method=orc.QUEST,
                            mode=orc.SEPARATE)
        assert r["cand"] == [1, 2]
        assert np.array_equal(r["scores"][0], c["quest_group_scores"]), (key, r["scores"])
        assert r["sel"][0] == c["sel"], key
        if key == "decode_step":
            assert np.array_equal(r["head_scores"], c["quest_head_scores"])
            for m, name in ((orc.MAX, "max_group_scores"), (orc.MEAN, "mean_group_scores")):
                rr = orc.decode_step(q, K, V, B=2, initial_len=2, local_len=2, topk=1, method=m)
                assert np.array_equal(rr["scores"][0], c[name]), (name, rr["scores"])
                assert rr["sel"][0] == c["sel"]


def check_regions_golden(orc):
    gd = golden()
    for c in gd["regions"]["cases"]:
        ie, ls, cand = orc.regions(c["L"], c["B"], c["I"], c["W"])
        assert (ie, ls) == (c["init_end"], c["local_start"]), c
        if "cand" in c:
            assert cand == c["cand"], c
        else:
            assert len(cand) == c["n_cand"] and cand[0] == ie // c["B"], c
    c = gd["kt_base_config_attended"]
    ie, ls, cand = orc.regions(c["L"], c["B"], c["I"], c["W"])
    sel = cand[: c["topk"]]
    toks = orc.attended_tokens(c["L"], c["B"], ie, ls, sel)
    assert len(toks) == c["attended_tokens"] == len(set(toks))


def check_regions_partition(orc):
    """Every token is Initial, in exactly one candidate block, or Local; candidates are full
    blocks; Local holds the partial last block."""
    for L in (1, 5, 127, 128, 129, 1000, 4096, 5000):
        for B in (4, 16, 128):
            for I in (0, 1, 100, 128, 300):
                for W in (0, 1, 100, 128, 1024):
                    ie, ls, cand = orc.regions(L, B, I, W)
                    cover = [0] * L
                    for t in range(ie):
                        cover[t] += 1
                    for b in cand:
                        assert (b + 1) * B <= L
                        for t in range(b * B, (b + 1) * B):
                            cover[t] += 1
                    for t in range(ls, L):
                        cover[t] += 1
                    assert all(c == 1 for c in cover), (L, B, I, W)
                    assert ie % B == 0 or ie == L
                    assert ls >= L - W - B + 1 or ls == ie
                    if L % B and L > ie:
                        assert ls <= (L // B) * B  # the partial last block is Local


# -------------------------------------------------------------------------------------- heads
def check_shared_is_sum_of_separate(orc, seed=5):
    q, K, V, _ = small_seq(seed, L=640, Hq=8, Hkv=2, d=16, B=16)
    for m in orc.REP_METHODS:
        reps = orc.block_reps(K, 16, m, rep_num=4)
        s = orc.head_scores(q, reps, m)
        sep = orc.group_scores(s, 2, orc.SEPARATE)
        sh = orc.group_scores(s, 2, orc.SHARED)
        assert sep.shape == (2, 40) and sh.shape == (1, 40)
        assert np.allclose(sh[0], sep.sum(axis=0), rtol=1e-12, atol=1e-12)
        # SEPARATE row h only depends on the query heads that read KV head h
        q2 = q.copy()
        q2[:4] = 0
        sep2 = orc.group_scores(orc.head_scores(q2, reps, m), 2, orc.SEPARATE)
        assert np.array_equal(sep2[1], sep[1]) and np.all(sep2[0] == 0)


def check_gqa_mapping_via_sdpa(orc, seed=6):
    """Dense attention (k >= n_cand) equals torch SDPA with enable_gqa (contiguous head groups)."""
    for (Hq, Hkv, L) in ((4, 2, 300), (8, 8, 129), (6, 3, 77), (8, 1, 200)):
        q, K, V, _ = small_seq(seed, L=L, Hq=Hq, Hkv=Hkv, d=16, B=16)
        r = orc.decode_step(q, K, V, B=16, initial_len=16, local_len=32, topk=10 ** 6,
                            method=orc.QUEST, mode=orc.SEPARATE)
        ref = F.scaled_dot_product_attention(
            torch.from_numpy(q.astype(np.float64))[None, :, None, :],
            torch.from_numpy(K.astype(np.float64)).permute(1, 0, 2)[None],
            torch.from_numpy(V.astype(np.float64)).permute(1, 0, 2)[None],
            enable_gqa=True)[0, :, 0, :].numpy()
        assert np.allclose(r["out"], ref, rtol=0, atol=1e-12), (Hq, Hkv, L)


def check_masked_attention_via_sdpa(orc, seed=8):
    """For an arbitrary selection, O6 equals SDPA with a boolean mask over exactly the attended set."""
    for mode in (orc.SEPARATE, orc.SHARED):
        q, K, V, _ = small_seq(seed, L=777, Hq=4, Hkv=2, d=16, B=16)
        r = orc.decode_step(q, K, V, B=16, initial_len=20, local_len=100, topk=5,
                            method=orc.MEAN, mode=mode)
        L = K.shape[0]
        mask = torch.zeros((1, 4, 1, L), dtype=torch.bool)
        g = 2
        for j in range(4):
            grp = (j // g) if mode == orc.SEPARATE else 0
            T = list(range(32)) + [t for b in r["sel"][grp] for t in range(16 * b, 16 * b + 16)] \
                + list(range(r["local_start"], L))
            mask[0, j, 0, T] = True
            assert sorted(r["tokens"][j]) == sorted(T)
        ref = F.scaled_dot_product_attention(
            torch.from_numpy(q.astype(np.float64))[None, :, None, :],
            torch.from_numpy(K.astype(np.float64)).permute(1, 0, 2)[None],
            torch.from_numpy(V.astype(np.float64)).permute(1, 0, 2)[None],
            attn_mask=mask, enable_gqa=True)[0, :, 0, :].numpy()
        assert np.allclose(r["out"], ref, rtol=0, atol=1e-12), mode


def check_softmax_identities(orc, seed=9):
    """q = 0 -> mean of the attended V rows; L = 1 -> V[0]; K[t] += a*q shifts every logit equally
    (output unchanged)."""
    q, K, V, _ = small_seq(seed, L=200, Hq=2, Hkv=1, d=16, B=16)
    q0 = np.zeros_like(q, dtype=np.float64)
    r = orc.decode_step(q0, K, V, B=16, initial_len=16, local_len=32, topk=3, method=orc.QUEST)
    for j in range(2):
        T = r["tokens"][j]
        assert np.allclose(r["out"][j], V[T, 0].astype(np.float64).mean(axis=0), atol=1e-13)
    r1 = orc.decode_step(q, K[:1], V[:1], B=16, initial_len=16, local_len=32, topk=3,
                         method=orc.QUEST)
    assert np.array_equal(r1["out"], np.repeat(V[:1, 0].astype(np.float64), 2, axis=0))
    qs = q[:1].astype(np.float64)
    Ks = K.astype(np.float64) + 0.75 * qs[0][None, None, :]
    toks = [list(range(200))]
    a = orc.attention(qs, K, V, toks)
    b = orc.attention(qs, Ks, V, toks)
    assert np.allclose(a, b, atol=1e-12)


def check_planted_recall(orc):
    """Hot blocks planted +2 along the query direction are what the selection picks (c1-like)."""
    B = 128
    L, I, W = 8192, 128, 1024
    for seed in (101, 102):
        s = kvsynth.make_sequence(seed, L, 8, 8, 128, B, hot_range=(1, 56), n_hot=4)
        for m in (orc.QUEST, orc.MAX, orc.MEAN):
            r = orc.decode_step(s.q.numpy(), s.K.numpy(), s.V.numpy(), B=B, initial_len=I,
                                local_len=W, topk=8, method=m, mode=orc.SEPARATE)
            for h in range(8):
                assert set(s.hot[h]) <= set(r["sel"][h]), (seed, m, h)


# ------------------------------------------------------------------------------------- Q8_0 cache
GOLDEN_Q8 = os.path.join(os.path.dirname(__file__), "golden", "q8_0_worked.json")


def check_q8_golden(orc):
    """The hand-worked Q8_0 blocks of tests/golden/q8_0_worked.json: scale, codes, cached values."""
    with open(GOLDEN_Q8) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = np.zeros(32, dtype=np.float32)
        for k, v in c["x_nonzero"].items():
            x[int(k)] = v
        codes, sc = orc.quantize_q8_0(x[None, :])
        assert float(sc[0, 0]) == c["d"], (c["why"], float(sc[0, 0]))
        want = np.zeros(32, dtype=np.int64)
        for k, v in c["codes_nonzero"].items():
            want[int(k)] = v
        assert np.array_equal(codes[0].astype(np.int64), want), (c["why"], codes[0])
        deq = orc.dequantize_q8_0(codes, sc)[0]
        wd = np.zeros(32)
        for k, v in c["deq_nonzero"].items():
            wd[int(k)] = v
        assert np.array_equal(deq, wd), (c["why"], deq)


def check_q8_error_bound_and_range(orc, seed=21):
    """On random rows: codes lie in [-127, 127]; each block's largest |x| takes code +-127; the
    fp32 reconstruction d*q is within d/2 of x (the rounding bound), and the cached value within
    d/2 + 127 |d - fp16(d)|; blocks are 32 channels wide (a block's scale ignores its neighbours)."""
    g = np.random.default_rng(seed)
    x = (g.standard_normal((64, 128)) * g.uniform(0.01, 30, (64, 1))).astype(np.float16).astype(np.float32)
    x[3, 32:64] = 0.0                           # one all-zero block
    x[5, :32] *= 1000.0                         # a loud block next to quiet ones
    codes, sc = orc.quantize_q8_0(x)
    assert codes.shape == x.shape and sc.shape == (64, 4)
    c = codes.astype(np.int64).reshape(64, 4, 32)
    xg = x.astype(np.float64).reshape(64, 4, 32)
    assert c.min() >= -127 and c.max() <= 127
    amax = np.abs(xg).max(axis=-1)
    d32 = (amax.astype(np.float32) / np.float32(127)).astype(np.float64)
    arg = np.abs(xg).argmax(axis=-1)
    top = np.take_along_axis(c, arg[..., None], -1)[..., 0]
    nz = amax > 0
    assert np.all(np.abs(top[nz]) == 127)
    assert np.all(c[~nz] == 0) and np.all(sc.astype(np.float64)[~nz] == 0)
    err32 = np.abs(xg - d32[..., None] * c)
    assert np.all(err32 <= d32[..., None] * (0.5 + 1e-5)), err32.max()
    deq = orc.dequantize_q8_0(codes, sc).reshape(64, 4, 32)
    d16 = sc.astype(np.float64)
    assert np.all(np.abs(xg - deq) <= (d32 * (0.5 + 1e-5) + 127 * np.abs(d32 - d16))[..., None])
    # the quiet blocks of row 5 keep their own scale
    assert np.all(sc[5, 1:].astype(np.float64) < sc[5, 0].astype(np.float64) / 100)


def check_q8_integer_rows_exact(orc):
    """Rows of integers whose blocks each hold +-127 are their own codes, with d = 1."""
    g = np.random.default_rng(22)
    x = g.integers(-127, 128, (8, 128)).astype(np.float32)
    x[:, ::32] = 127.0
    codes, sc = orc.quantize_q8_0(x)
    assert np.all(sc.astype(np.float64) == 1.0)
    assert np.array_equal(codes.astype(np.float32), x)
    assert np.array_equal(orc.dequantize_q8_0(codes, sc), x.astype(np.float64))


GOLDEN_I8 = os.path.join(os.path.dirname(__file__), "golden", "int8_pth_worked.json")


def check_int8_pth_golden(orc):
    """The hand-worked rows of tests/golden/int8_pth_worked.json: fp32 scale, codes, cached values."""
    with open(GOLDEN_I8) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = np.zeros(128, dtype=np.float32)
        for k, v in c["x_nonzero"].items():
            x[int(k)] = v
        codes, s = orc.quantize_int8_pth(x[None])
        assert s.dtype == np.float32 and float(s[0]) == c["s"], (c["why"], float(s[0]))
        want = np.zeros(128, dtype=np.int64)
        for k, v in c["codes_nonzero"].items():
            want[int(k)] = v
        assert np.array_equal(codes[0].astype(np.int64), want), c["why"]
        deq = np.zeros(128)
        for k, v in c["deq_nonzero"].items():
            deq[int(k)] = v
        assert np.array_equal(orc.dequantize_int8_pth(codes, s)[0], deq), c["why"]


def check_int8_pth_bound_and_range(orc):
    """On random fp16 rows: codes in [-127, 127], each row's largest |x| takes +-127, the cached
    value is within s/2 (plus fp32 rounding) of x; integer rows holding +-127 are their own codes."""
    g = np.random.default_rng(27)
    x = kvsynth.randn_fp16((16, 4, 128), 27).numpy().astype(np.float32) * np.float32(3.0)
    x = x.astype(np.float16).astype(np.float32)
    codes, s = orc.quantize_int8_pth(x)
    assert codes.shape == x.shape and s.shape == x.shape[:-1]
    assert np.abs(codes.astype(np.int64)).max() <= 127
    top = np.take_along_axis(codes, np.abs(x).argmax(axis=-1)[..., None], -1)[..., 0]
    assert np.all(np.abs(top.astype(np.int64)) == 127)
    err = np.abs(orc.dequantize_int8_pth(codes, s) - x.astype(np.float64))
    bound = s.astype(np.float64)[..., None] * (0.5 + 1e-6) + np.abs(x) * 2.0 ** -23
    assert np.all(err <= bound)
    xi = g.integers(-127, 128, (8, 128)).astype(np.float32)
    xi[:, 17] = -127.0
    ci, si = orc.quantize_int8_pth(xi)
    assert np.all(si == 1.0) and np.array_equal(ci.astype(np.float32), xi)


GOLDEN_I4 = os.path.join(os.path.dirname(__file__), "golden", "int4_pth_worked.json")


def check_int4_pth_golden(orc):
    """The hand-worked rows of tests/golden/int4_pth_worked.json: fp32 scale, zero point, codes and
    cached values."""
    with open(GOLDEN_I4) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = np.full(128, c.get("fill", 0.0), dtype=np.float32)
        for k, v in c["x_nonzero"].items():
            x[int(k)] = v
        codes, s, z = orc.quantize_int4_pth(x[None])
        assert s.dtype == np.float32 and float(s[0]) == c["s"], (c["why"], float(s[0]))
        assert int(z[0]) == c["z"], (c["why"], int(z[0]))
        want = np.full(128, c["fill_code"], dtype=np.int64)
        for k, v in c["codes"].items():
            want[int(k)] = v
        assert np.array_equal(codes[0].astype(np.int64), want), c["why"]
        deq = np.full(128, c.get("deq_fill", 0.0))
        for k, v in c["deq_nonzero"].items():
            deq[int(k)] = v
        assert np.array_equal(orc.dequantize_int4_pth(codes, s, z)[0], deq), c["why"]


def check_int4_pth_bound_and_range(orc):
    """On random fp16 rows: codes and zero points in 0..15, every 0 cached as 0, the row's extremes
    reach the ends of the code range, and each cached value is within s/2 of x (within s where
    rounding clamped the code), plus fp32 rounding; integer rows of range 15 holding 0 are exact."""
    g = np.random.default_rng(28)
    x = kvsynth.randn_fp16((16, 4, 128), 28).numpy().astype(np.float32) * np.float32(3.0)
    x = x.astype(np.float16).astype(np.float32)
    x[0, 0, :] = np.abs(x[0, 0, :])  # rows without negative and without positive values
    x[1, 1, :] = -np.abs(x[1, 1, :])
    x[2, 2, 5] = 0.0
    codes, s, z = orc.quantize_int4_pth(x)
    assert codes.shape == x.shape and s.shape == x.shape[:-1] and z.shape == x.shape[:-1]
    assert codes.max() <= 15 and z.max() <= 15
    deq = orc.dequantize_int4_pth(codes, s, z)
    assert np.all(deq[x == 0] == 0)
    lo = np.minimum(x.min(axis=-1), 0)
    hi = np.maximum(x.max(axis=-1), 0)
    assert np.all(codes[x == hi[..., None]] >= 14) and np.all(codes[x == lo[..., None]] <= 1)
    t = x.astype(np.float64) / s.astype(np.float64)[..., None] + z.astype(np.float64)[..., None]
    clamped = (t > 15.5) | (t < -0.5)
    err = np.abs(deq - x.astype(np.float64))
    sc = s.astype(np.float64)[..., None]
    slack = np.abs(x) * 2.0 ** -20 + sc * 1e-6
    assert np.all(np.where(clamped, err <= sc + slack, err <= 0.5 * sc + slack))
    xi = g.integers(-7, 9, (8, 128)).astype(np.float32)
    xi[:, 3], xi[:, 4], xi[:, 5] = -7.0, 8.0, 0.0
    ci, si, zi = orc.quantize_int4_pth(xi)
    assert np.all(si == 1.0) and np.all(zi == 7)
    assert np.array_equal(orc.dequantize_int4_pth(ci, si, zi), xi.astype(np.float64))


GOLDEN_REPS = os.path.join(os.path.dirname(__file__), "golden", "stored_reps_worked.json")


def check_stored_reps_golden(orc):
    """The hand-worked values of tests/golden/stored_reps_worked.json: reps over a quantized cache are
    stored in fp16 with round-to-nearest-even (ties to even, also in the subnormal range), Mean in
    fp32; and whole Q8_0 / INT8 key tiles quantized, read back and reduced to those stored reps."""
    with open(GOLDEN_REPS) as f:
        gold = json.load(f)
    for c in gold["direct"]:
        got = orc.stored_reps(np.array([c["rep"]], dtype=np.float64), c["method"])
        assert got.shape == (1,) and float(got[0]) == c["stored"], (c["why"], float(got[0]))
    quant = {"q8_0": (orc.quantize_q8_0, orc.dequantize_q8_0),
             "int8_pth": (orc.quantize_int8_pth, orc.dequantize_int8_pth)}
    for c in gold["block"]:
        x = np.zeros((128, 128), dtype=np.float32)
        for t, row in c["x"].items():
            for ch, v in row.items():
                x[int(t), int(ch)] = v
        qf, df = quant[c["kv_type"]]
        K = df(*qf(x))[:, None, :]  # [128 tokens][1 KV head][128]
        for method, want in (("max", [c["max"]]), ("mean", [c["mean"]]),
                             ("quest", [c["quest_min"], c["quest_max"]])):
            got = orc.stored_reps(orc.block_reps(K, 128, method, 1), method)
            assert got.shape == (1, 1, len(want), 128), (c["kv_type"], method, got.shape)
            for r, w in enumerate(want):
                assert got[0, 0, r, :2].tolist() == w, (c["kv_type"], method, r, got[0, 0, r, :2], c["why"])
            assert np.all(got[0, 0, :, 2:] == 0.0), (c["kv_type"], method)


GOLDEN_Q4 = os.path.join(os.path.dirname(__file__), "golden", "q4_0_worked.json")


def check_q4_golden(orc):
    """The hand-worked Q4_0 blocks of tests/golden/q4_0_worked.json: scale (with its sign), codes,
    cached values."""
    with open(GOLDEN_Q4) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = np.zeros(32, dtype=np.float32)
        for k, v in c["x_nonzero"].items():
            x[int(k)] = v
        codes, sc = orc.quantize_q4_0(x[None, :])
        d = float(sc[0, 0])
        assert d == c["d"] and math.copysign(1.0, d) == math.copysign(1.0, c["d"]), (c["why"], d)
        for k, v in c["codes"].items():
            assert int(codes[0, int(k)]) == v, (c["why"], k, int(codes[0, int(k)]))
        deq = orc.dequantize_q4_0(codes, sc)[0]
        wd = np.zeros(32)
        for k, v in c["deq_nonzero"].items():
            wd[int(k)] = v
        assert np.array_equal(deq, wd), (c["why"], deq)


def check_q4_range_and_bound(orc, seed=23):
    """On random rows: codes in 0..15; each block's first largest-magnitude value takes code 0 and is
    reproduced up to the fp16 rounding of d; every value lies within |d| of x (within |d|/2 unless
    clipped at code 15); blocks are 32 channels wide."""
    g = np.random.default_rng(seed)
    x = (g.standard_normal((64, 128)) * g.uniform(0.01, 30, (64, 1))).astype(np.float16).astype(np.float32)
    x[5, :32] *= 1000.0
    codes, sc = orc.quantize_q4_0(x)
    c = codes.astype(np.int64).reshape(64, 4, 32)
    xg = x.astype(np.float64).reshape(64, 4, 32)
    assert c.min() >= 0 and c.max() <= 15
    first = np.abs(xg).argmax(axis=-1)
    assert np.all(np.take_along_axis(c, first[..., None], -1) == 0)
    m = np.take_along_axis(xg, first[..., None], -1)[..., 0]
    d32 = (m.astype(np.float32) / np.float32(-8)).astype(np.float64)
    err = np.abs(xg - d32[..., None] * (c - 8))
    tol = np.abs(d32)[..., None]
    assert np.all(err <= tol * (1 + 1e-6)), err.max()
    half = np.broadcast_to(tol / 2 * (1 + 1e-5), err.shape)
    assert np.all(err[c < 15] <= half[c < 15])
    assert np.all(np.abs(sc[5, 1:].astype(np.float64)) < np.abs(sc[5, 0].astype(np.float64)) / 100)


# ---------------------------------------------------------------------------------- Dynamic reps
def check_importance_via_sdpa(orc, seed=31):
    """Token importance = column sums of the attention probabilities, taken from torch's float64
    scaled_dot_product_attention with V = the identity (its output rows are the probabilities) and a
    causal mask offset to the observation window's positions."""
    g = np.random.default_rng(seed)
    for (L, Hq, Hkv, n, mode) in [(37, 4, 2, 5, "separate"), (50, 6, 3, 50, "shared"), (9, 2, 2, 1, "separate")]:
        d = 16
        K = g.standard_normal((L, Hkv, d)).astype(np.float16)
        q = (2 * g.standard_normal((n, Hq, d))).astype(np.float16)
        imp = orc.token_importance(q, K, mode)
        grp = Hq // Hkv
        eye = torch.eye(L, dtype=torch.float64)
        pos = torch.arange(L - n, L)[:, None]
        mask = torch.arange(L)[None, :] <= pos  # [n][L]
        want = np.zeros((Hkv, L))
        for j in range(Hq):
            h = j // grp
            Q = torch.tensor(q[:, j, :], dtype=torch.float64)[None, None]
            Kt = torch.tensor(K[:, h, :], dtype=torch.float64)[None, None]
            P = F.scaled_dot_product_attention(Q, Kt, eye[None, None], attn_mask=mask[None, None])[0, 0]
            want[h] += P.sum(dim=0).numpy()
        if mode == "shared":
            want = want.sum(axis=0, keepdims=True)
        assert np.allclose(imp, want, rtol=1e-12, atol=1e-12), np.abs(imp - want).max()


def check_importance_mass_and_causality(orc, seed=32):
    """Each observation query spreads one unit of attention per query head over the keys it may see,
    so a group's importance sums to n_obs times its query heads; SHARED is the sum of SEPARATE; with
    q = 0 every visible key gets 1/(position + 1) from each query, and a key inside the window only
    from the queries at or after it."""
    g = np.random.default_rng(seed)
    L, Hq, Hkv, n, d = 60, 8, 2, 7, 16
    K = g.standard_normal((L, Hkv, d)).astype(np.float16)
    q = g.standard_normal((n, Hq, d)).astype(np.float16)
    imp = orc.token_importance(q, K, "separate")
    assert np.allclose(imp.sum(axis=1), n * (Hq // Hkv), rtol=1e-12)
    shared = orc.token_importance(q, K, "shared")
    assert np.allclose(shared[0], imp.sum(axis=0), rtol=1e-12)
    # q = 0: uniform weights, so key t gets sum over the queries that see it of 1/(position+1)
    z = orc.token_importance(np.zeros_like(q), K, "separate")
    for t in range(L):
        want = sum(1.0 / (L - n + i + 1) for i in range(n) if t <= L - n + i) * (Hq // Hkv)
        assert abs(z[0, t] - want) < 1e-12, (t, z[0, t], want)


def check_dynamic_reps_closed_forms(orc, seed=33):
    """rep_num = B takes every row; uniform importance (q = 0, a block before the window) takes the
    block's first rep_num rows in order; a key planted along every observation query is taken."""
    g = np.random.default_rng(seed)
    L, Hq, Hkv, n, d, B = 64, 4, 2, 4, 16, 8
    K = g.standard_normal((L, Hkv, d)).astype(np.float16)
    q = g.standard_normal((n, Hq, d)).astype(np.float16)
    imp = orc.token_importance(q, K, "separate")
    allr, picked = orc.dynamic_reps(K, imp, B, B, "separate", [2, 5])
    assert np.array_equal(allr[0], np.asarray(K[16:24], np.float64).transpose(1, 0, 2))
    z = orc.token_importance(np.zeros_like(q), K, "shared")
    r, p = orc.dynamic_reps(K, z, B, 3, "shared", [1, 3])
    assert p.tolist() == [[[0, 1, 2]] * Hkv] * 2
    assert np.array_equal(r[0, :, 0], np.asarray(K[8], np.float64))
    K2 = K.copy()
    K2[8 * 4 + 5, 1, :] = (8.0 * np.sign(q[:, 2:4, :].astype(np.float64).sum(axis=(0, 1)))).astype(np.float16)
    imp2 = orc.token_importance(q, K2, "separate")
    _, p2 = orc.dynamic_reps(K2, imp2, B, 2, "separate", [4])
    assert 5 in p2[0, 1].tolist(), p2


# ---------------------------------------------------------------------------------------- Preselect
def check_preselect_identities(orc, seed=34):
    """A set holding every candidate leaves the decode step as it is; with k >= the set's size the
    set itself is attended; a block whose tokens all take the largest scores is preselected; the set
    is the candidates ranked by summed token score (a block-sum reference written as a matrix
    product)."""
    g = np.random.default_rng(seed)
    L, Hq, Hkv, d, B, I, W = 60 * 8 + 5, 4, 2, 16, 8, 8, 24
    q = g.standard_normal((Hq, d)).astype(np.float16)
    K = g.standard_normal((L, Hkv, d)).astype(np.float16)
    V = g.standard_normal((L, Hkv, d)).astype(np.float16)
    _, _, cand = orc.regions(L, B, I, W)
    kw = dict(B=B, initial_len=I, local_len=W, method="quest", mode="separate")
    full = orc.decode_step(q, K, V, topk=6, **kw)
    allp = orc.decode_step_preselected(q, K, V, [cand] * Hkv, topk=6, **kw)
    assert allp["sel"] == full["sel"] and np.array_equal(allp["out"], full["out"])
    presel = [cand[3:9], cand[10:14]]
    r = orc.decode_step_preselected(q, K, V, presel, topk=10, **kw)
    assert r["sel"] == presel
    r2 = orc.decode_step_preselected(q, K, V, presel, topk=2, **kw)
    for gi in range(Hkv):
        assert set(r2["sel"][gi]) <= set(presel[gi]) and len(r2["sel"][gi]) == 2
    imp = np.abs(g.standard_normal((Hkv, L)))
    imp[1, 20 * B:21 * B] += 50.0
    ps = orc.preselect_blocks(imp, L, B, I, W, 5)
    assert 20 in ps[1] and all(len(p) == 5 and p == sorted(p) for p in ps)
    M = np.zeros((L, len(cand)))
    for j, b in enumerate(cand):
        M[b * B:(b + 1) * B, j] = 1.0
    bs = imp @ M
    for gi in range(Hkv):
        order = sorted(range(len(cand)), key=lambda j: (-bs[gi, j], cand[j]))[:5]
        assert ps[gi] == sorted(cand[j] for j in order)


def _pseudocode_preselect(imp_row, lo, hi, B, pool_kernel, n_presel):
    """The pooled preselect as the article's pseudocode orders it: torch's avg_pool1d over the
    Context votes, tokens in descending pooled vote (ties to the lower token), blocks collected in
    that order until n_presel distinct ones are hit."""
    import torch
    v = torch.tensor(imp_row[lo:hi], dtype=torch.float64)[None, None]
    pv = torch.nn.functional.avg_pool1d(v, pool_kernel, stride=1, padding=pool_kernel // 2,
                                        count_include_pad=True)[0, 0].numpy()
    order = sorted(range(hi - lo), key=lambda t: (-pv[t], t))
    got = []
    for t in order:
        b = (lo + t) // B
        if b not in got:
            got.append(b)
        if len(got) == n_presel:
            break
    return sorted(got), pv


def check_preselect_pooled(orc, seed=35):
    """Pooled preselect (reading R26): the pooled votes are torch's avg_pool1d of the Context slice;
    the set is what the pseudocode's token ranking hits first; a vote spike pools into the next
    block; votes of Initial / Local tokens are not pooled into the Context; pool_kernel = 1 ranks
    blocks by their largest token score."""
    g = np.random.default_rng(seed)
    L, B, I, W = 50 * 8 + 3, 8, 8, 24
    lo, hi, cand = orc.regions(L, B, I, W)
    imp = np.abs(g.standard_normal((3, L)))
    for pk, n in ((5, 7), (7, 3), (3, 12), (9, 1), (127, 4)):  # 127: the widest window the ABI takes
        got = orc.preselect_blocks(imp, L, B, I, W, n, pool_kernel=pk)
        for gi in range(3):
            want, pv = _pseudocode_preselect(imp[gi], lo, hi, B, pk, n)
            assert got[gi] == want, (pk, n, gi, got[gi], want)
            assert np.allclose(orc.pooled_votes(imp[gi], lo, hi, pk), pv, rtol=1e-13, atol=0)
    got1 = orc.preselect_blocks(imp, L, B, I, W, 6, pool_kernel=1)
    mx = imp[:, lo:hi].reshape(3, -1, B).max(axis=-1)
    for gi in range(3):
        order = sorted(range(len(cand)), key=lambda j: (-mx[gi, j], cand[j]))[:6]
        assert got1[gi] == sorted(cand[j] for j in order)
    # a spike on the last token of block 20 lifts block 21 through the window, not block 19
    sp = 1e-3 * np.abs(g.standard_normal((1, L)))
    sp[0, 21 * B - 1] = 10.0
    assert orc.preselect_blocks(sp, L, B, I, W, 2, pool_kernel=5) == [[20, 21]]
    assert orc.preselect_blocks(sp, L, B, I, W, 1, pool_kernel=0) == [[20]]
    # spikes on the last Initial and first Local tokens stay outside the Context's pooling
    edge = 1e-3 * np.abs(g.standard_normal((1, L)))
    edge[0, lo - 1] = edge[0, hi] = 10.0
    edge[0, 30 * B:31 * B] = 1.0
    assert orc.preselect_blocks(edge, L, B, I, W, 1, pool_kernel=7) == [[30]]


ALL_CHECKS = [
    check_quest_upper_bound, check_quest_tight_and_units, check_rep_closed_forms,
    check_hand_worked, check_regions_golden, check_regions_partition,
    check_shared_is_sum_of_separate, check_gqa_mapping_via_sdpa, check_masked_attention_via_sdpa,
    check_softmax_identities, check_q8_golden, check_q8_error_bound_and_range,
    check_q8_integer_rows_exact, check_importance_via_sdpa, check_importance_mass_and_causality,
    check_dynamic_reps_closed_forms, check_preselect_identities, check_q4_golden,
    check_q4_range_and_bound, check_preselect_pooled, check_int8_pth_golden,
    check_int8_pth_bound_and_range, check_int4_pth_golden, check_int4_pth_bound_and_range,
    check_stored_reps_golden,
]
