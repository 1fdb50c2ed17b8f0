"""The oracle against what the pages and the mathematics fix (CPU only)."""
import math

import numpy as np
import pytest

import oracle_checks as oc
from oracle import kvs_oracle as orc


@pytest.mark.parametrize("check", oc.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(orc)


def test_planted_recall():
    oc.check_planted_recall(orc)


# ------------------------------------------------------------------------------------------------
# Mutation tests: plant a plausible mistake in the oracle and show that some pin fails.
# ------------------------------------------------------------------------------------------------
def _quest_kmax_only(q, reps, method):
    s = _orig_head_scores(q, reps, method)
    if method == orc.QUEST:
        Hq = q.shape[0]
        g = Hq // reps.shape[1]
        for j in range(Hq):
            s[:, j] = (np.asarray(q[j], np.float64) * reps[:, j // g, 1, :]).sum(axis=1)
    return s


def _quest_min_of_products(q, reps, method):
    s = _orig_head_scores(q, reps, method)
    if method == orc.QUEST:
        Hq = q.shape[0]
        g = Hq // reps.shape[1]
        for j in range(Hq):
            qj = np.asarray(q[j], np.float64)
            s[:, j] = np.minimum(qj * reps[:, j // g, 1], qj * reps[:, j // g, 0]).sum(axis=1)
    return s


def _dropped_channel(q, reps, method):
    q = np.array(q, dtype=np.float64)
    q[:, -1] = 0.0
    return _orig_head_scores(q, reps, method)


def _gqa_modulo(q, reps, method):
    q = np.asarray(q, dtype=np.float64)
    Hq, Hkv = q.shape[0], reps.shape[1]
    s = np.empty((reps.shape[0], Hq))
    for j in range(Hq):
        h = j % Hkv  # wrong: interleaved instead of contiguous groups
        if method == orc.QUEST:
            s[:, j] = np.maximum(q[j] * reps[:, h, 1], q[j] * reps[:, h, 0]).sum(axis=1)
        else:
            s[:, j] = (reps[:, h] * q[j]).sum(axis=(1, 2))
    return s


def _ties_high_index(scores_row, cand, k):
    ranked = sorted(range(len(cand)), key=lambda i: (-scores_row[i], -cand[i]))
    return sorted(cand[i] for i in ranked[:min(k, len(cand))])


def _local_one_block_short(L, B, initial_len, local_len):
    ie, ls, cand = _orig_regions(L, B, initial_len, local_len)
    if cand:
        return ie, ls + B, cand + [ls // B] if (ls + B) <= L else cand
    return ie, ls, cand


def _attention_no_scale(q, K, V, toks, scale=None):
    return _orig_attention(q, K, V, toks, scale=1.0)


def _mean_wrong_divisor(K, B, method, rep_num=1, blocks=None):
    r = _orig_block_reps(K, B, method, rep_num, blocks)
    if method == orc.MEAN:
        r = r * B / (B - 1)
    return r


def _fix_wrong_offset(K, B, method, rep_num=1, blocks=None):
    if method != orc.FIX:
        return _orig_block_reps(K, B, method, rep_num, blocks)
    L, Hkv, d = K.shape
    blocks = list(range(L // B)) if blocks is None else list(blocks)
    stride = B // rep_num
    out = np.empty((len(blocks), Hkv, rep_num, d))
    for i, b in enumerate(blocks):
        for r in range(rep_num):
            out[i, :, r] = K[b * B + r * stride + stride - 1]
    return out


def _shared_as_mean(s, Hkv, mode):
    r = _orig_group_scores(s, Hkv, mode)
    return r / s.shape[1] if mode == orc.SHARED else r


def _q8_round_half_even(x):
    codes, sc = _orig_quantize(x)
    x = np.asarray(x, dtype=np.float32)
    *lead, d = x.shape
    xg = x.reshape(*lead, d // 32, 32)
    dsc = (np.abs(xg).max(axis=-1) / np.float32(127)).astype(np.float32)
    inv = np.where(dsc != 0, np.float32(1) / np.where(dsc != 0, dsc, 1), 0).astype(np.float32)
    v = (xg * inv[..., None]).astype(np.float32)
    return np.round(v).astype(np.int8).reshape(*lead, d), sc


def _q8_scale_128(x):
    x = np.asarray(x, dtype=np.float32)
    *lead, d = x.shape
    xg = x.reshape(*lead, d // 32, 32)
    dsc = (np.abs(xg).max(axis=-1) / np.float32(128)).astype(np.float32)
    inv = np.where(dsc != 0, np.float32(1) / np.where(dsc != 0, dsc, 1), 0).astype(np.float32)
    v = (xg * inv[..., None]).astype(np.float64)
    codes = np.clip(np.sign(v) * np.floor(np.abs(v) + 0.5), -128, 127)
    return codes.astype(np.int8).reshape(*lead, d), dsc.astype(np.float16)


def _q8_block_16(x):
    """Codes scaled per 16 channels, reported with the scale of each 32-channel block's first half."""
    x = np.asarray(x, dtype=np.float32)
    *lead, d = x.shape
    xg = x.reshape(*lead, d // 16, 16)
    dsc = (np.abs(xg).max(axis=-1) / np.float32(127)).astype(np.float32)
    inv = np.where(dsc != 0, np.float32(1) / np.where(dsc != 0, dsc, 1), 0).astype(np.float32)
    v = (xg * inv[..., None]).astype(np.float64)
    codes = (np.sign(v) * np.floor(np.abs(v) + 0.5)).astype(np.int8).reshape(*lead, d)
    return codes, dsc.reshape(*lead, d // 32, 2)[..., 0].astype(np.float16)


def _q8_deq_fp32_scale(codes, scales):
    return _orig_dequantize(codes, scales) * 1.0001


def _importance_not_causal(q_obs, K, mode, scale=None):
    n = q_obs.shape[0]
    Kp = K
    q64 = np.asarray(q_obs, np.float64)
    L, Hkv, d = K.shape
    g = q64.shape[1] // Hkv
    imp = np.zeros((Hkv, L))
    for h in range(Hkv):
        for i in range(n):
            for j in range(h * g, (h + 1) * g):
                z = (np.asarray(Kp[:, h], np.float64) @ q64[i, j]) / math.sqrt(d)
                w = np.exp(z - z.max())
                imp[h] += w / w.sum()
    return imp if mode == orc.SEPARATE else imp.sum(axis=0, keepdims=True)


def _dynamic_ties_high(K, imp, B, rep_num, mode, blocks):
    L, Hkv, d = K.shape
    blocks = list(blocks)
    out = np.empty((len(blocks), Hkv, rep_num, d))
    picked = np.empty((len(blocks), Hkv, rep_num), dtype=np.int64)
    for n, b in enumerate(blocks):
        for h in range(Hkv):
            row = imp[h if mode == orc.SEPARATE else 0, b * B:(b + 1) * B]
            toks = sorted(sorted(range(B), key=lambda t: (-row[t], -t))[:rep_num])
            picked[n, h] = toks
            out[n, h] = np.asarray(K[[b * B + t for t in toks], h, :], np.float64)
    return out, picked


def _presel_max_not_sum(imp, L, B, initial_len, local_len, n_presel):
    _, _, cand = orc.regions(L, B, initial_len, local_len)
    return [orc.select_topk([row[b * B:(b + 1) * B].max() for b in cand], cand, n_presel)
            for row in np.asarray(imp, np.float64)]


def _i8_generic(x, even=False, div=127.0, group=128, half_scale=False):
    x = np.asarray(x, dtype=np.float32)
    *lead, d = x.shape
    xg = x.reshape(*lead, d // group, group)
    s = (np.abs(xg).max(axis=-1) / np.float32(div)).astype(np.float32)
    if half_scale:
        s = s.astype(np.float16).astype(np.float32)
    inv = np.where(s != 0, np.float32(1) / np.where(s != 0, s, 1), 0).astype(np.float32)
    v = (xg * inv[..., None]).astype(np.float32).astype(np.float64)
    q = np.round(v) if even else np.sign(v) * np.floor(np.abs(v) + 0.5)
    codes = q.astype(np.int8).reshape(*lead, d)
    return codes, (s[..., 0] if group == 128 else s.max(axis=-1))


def _i8_round_even(x):
    return _i8_generic(x, even=True)


def _i8_div_128(x):
    return _i8_generic(x, div=128.0)


def _i8_block_32(x):
    return _i8_generic(x, group=32)


def _i8_fp16_scale(x):
    return _i8_generic(x, half_scale=True)


def _i4_generic(x, away=False, zero_in_range=True, clamp=True, symmetric=False, half_scale=False):
    x = np.asarray(x, dtype=np.float32)
    lo, hi = x.min(axis=-1), x.max(axis=-1)
    if zero_in_range:
        lo, hi = np.minimum(lo, 0).astype(np.float32), np.maximum(hi, 0).astype(np.float32)
    if symmetric:
        s = (np.maximum(np.abs(lo), np.abs(hi)) / np.float32(7.0)).astype(np.float32)
    else:
        s = ((hi - lo).astype(np.float32) / np.float32(15.0)).astype(np.float32)
    if half_scale:
        s = s.astype(np.float16).astype(np.float32)
    inv = np.where(s != 0, np.float32(1) / np.where(s != 0, s, 1), 0).astype(np.float32)
    rnd = (lambda v: np.sign(v) * np.floor(np.abs(v) + 0.5)) if away else np.rint
    z = np.full(s.shape, 8.0) if symmetric else rnd((-lo * inv).astype(np.float32).astype(np.float64))
    z = np.where(s != 0, np.clip(z, 0, 15), 0).astype(np.int64)
    t = rnd((x * inv[..., None]).astype(np.float32).astype(np.float64)).astype(np.int64) + z[..., None]
    codes = (np.clip(t, 0, 15) if clamp else t & 15).astype(np.uint8)
    return codes, s, z.astype(np.uint8)


def _i4_ties_away(x):
    return _i4_generic(x, away=True)


def _i4_range_without_zero(x):
    return _i4_generic(x, zero_in_range=False)


def _i4_wraps_instead_of_clamp(x):
    return _i4_generic(x, clamp=False)


def _i4_symmetric(x):
    return _i4_generic(x, symmetric=True)


def _i4_fp16_scale(x):
    return _i4_generic(x, half_scale=True)


def _i4_dequant_drops_zero_point(codes, scales, zeros):
    c = np.asarray(codes, dtype=np.int64)
    return (c.astype(np.float32) * np.asarray(scales, np.float32)[..., None]).astype(np.float32).astype(np.float64)


_orig_preselect = orc.preselect_blocks


def _presel_pooled_variant(kind):
    """Pooled preselect with one plausible mistake: pooling inside each block only, pooling over the
    whole row (Initial / Local votes leak in), or a block's pooled votes summed instead of maxed."""
    def f(imp, L, B, initial_len, local_len, n_presel, pool_kernel=0):
        if pool_kernel == 0:
            return _orig_preselect(imp, L, B, initial_len, local_len, n_presel)
        lo, hi, cand = orc.regions(L, B, initial_len, local_len)
        h = pool_kernel // 2
        out = []
        for row in np.asarray(imp, np.float64):
            bs = []
            for b in cand:
                a, e = (b * B, (b + 1) * B) if kind == "in_block" else ((0, L) if kind == "full_row" else (lo, hi))
                pv = [sum(row[u] for u in range(t - h, t + h + 1) if a <= u < e) / pool_kernel
                      for t in range(b * B, (b + 1) * B)]
                bs.append(sum(pv) if kind == "sum" else max(pv))
            out.append(orc.select_topk(bs, cand, n_presel))
        return out
    f.__name__ = f"_presel_pool_{kind}"
    return f


def _presel_decode_ignores_set(q, K, V, presel, **kw):
    return orc.decode_step(q, K, V, **kw)


def _q4_generic(x, last=False, rne=False, clip=True):
    x = np.asarray(x, dtype=np.float32)
    *lead, d = x.shape
    xg = x.reshape(*lead, d // 32, 32)
    a = np.abs(xg)
    idx = (31 - a[..., ::-1].argmax(axis=-1)) if last else a.argmax(axis=-1)
    m = np.take_along_axis(xg, idx[..., None], -1)[..., 0]
    dsc = (m / np.float32(-8)).astype(np.float32)
    inv = np.where(dsc != 0, np.float32(1) / np.where(dsc != 0, dsc, 1), 0).astype(np.float32)
    v = (xg * inv[..., None]).astype(np.float32)
    q = (np.round(v.astype(np.float64)) + 8) if rne else np.trunc((v + np.float32(8.5)).astype(np.float64))
    q = np.minimum(15, q) if clip else q
    return q.astype(np.uint8).reshape(*lead, d), dsc.astype(np.float16)


def _q4_last_max(x):
    return _q4_generic(x, last=True)


def _q4_round_even(x):
    return _q4_generic(x, rne=True)


def _q4_no_clip(x):
    return _q4_generic(x, clip=False)


def _fp16_toward_zero(x):
    x = np.asarray(x, dtype=np.float64)
    h = x.astype(np.float16)
    over = np.abs(h.astype(np.float64)) > np.abs(x)
    return np.where(over, np.nextafter(h, np.float16(0)), h).astype(np.float64)


def _stored_reps_truncated(reps, method):
    if method == orc.MEAN:
        return _orig_stored_reps(reps, method)
    return _fp16_toward_zero(reps)


def _stored_reps_mean_fp16(reps, method):
    return np.asarray(reps, dtype=np.float64).astype(np.float16).astype(np.float64)


def _stored_reps_ties_away(reps, method):
    if method == orc.MEAN:
        return _orig_stored_reps(reps, method)
    x = np.asarray(reps, dtype=np.float64)
    lo = _fp16_toward_zero(x)
    hi = np.nextafter(lo.astype(np.float16), np.copysign(np.float16(np.inf), x).astype(np.float16)).astype(np.float64)
    tie = (x - lo) == (hi - x)
    return np.where(tie & (lo != x), hi, x.astype(np.float16).astype(np.float64))


_orig_quantize = orc.quantize_q8_0
_orig_dequantize = orc.dequantize_q8_0
_orig_head_scores = orc.head_scores
_orig_select = orc.select_topk
_orig_regions = orc.regions
_orig_attention = orc.attention
_orig_block_reps = orc.block_reps
_orig_group_scores = orc.group_scores
_orig_stored_reps = orc.stored_reps

MUTANTS = [
    ("head_scores", _quest_kmax_only),
    ("head_scores", _quest_min_of_products),
    ("head_scores", _dropped_channel),
    ("head_scores", _gqa_modulo),
    ("select_topk", _ties_high_index),
    ("regions", _local_one_block_short),
    ("attention", _attention_no_scale),
    ("block_reps", _mean_wrong_divisor),
    ("block_reps", _fix_wrong_offset),
    ("group_scores", _shared_as_mean),
    ("quantize_q8_0", _q8_round_half_even),
    ("quantize_q8_0", _q8_scale_128),
    ("quantize_q8_0", _q8_block_16),
    ("dequantize_q8_0", _q8_deq_fp32_scale),
    ("token_importance", _importance_not_causal),
    ("dynamic_reps", _dynamic_ties_high),
    ("preselect_blocks", _presel_max_not_sum),
    ("quantize_q4_0", _q4_last_max),
    ("quantize_q4_0", _q4_round_even),
    ("quantize_q4_0", _q4_no_clip),
    ("decode_step_preselected", _presel_decode_ignores_set),
    ("preselect_blocks", _presel_pooled_variant("in_block")),
    ("preselect_blocks", _presel_pooled_variant("full_row")),
    ("preselect_blocks", _presel_pooled_variant("sum")),
    ("quantize_int8_pth", _i8_round_even),
    ("quantize_int8_pth", _i8_div_128),
    ("quantize_int8_pth", _i8_block_32),
    ("quantize_int8_pth", _i8_fp16_scale),
    ("quantize_int4_pth", _i4_ties_away),
    ("quantize_int4_pth", _i4_range_without_zero),
    ("quantize_int4_pth", _i4_wraps_instead_of_clamp),
    ("quantize_int4_pth", _i4_symmetric),
    ("quantize_int4_pth", _i4_fp16_scale),
    ("dequantize_int4_pth", _i4_dequant_drops_zero_point),
    ("stored_reps", _stored_reps_truncated),
    ("stored_reps", _stored_reps_mean_fp16),
    ("stored_reps", _stored_reps_ties_away),
]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_pins_catch_mutant(monkeypatch, name, mutant):
    import test_oracle_bruteforce as bf
    monkeypatch.setattr(orc, name, mutant)
    failed = []
    for check in oc.ALL_CHECKS + [bf.check_against_bruteforce]:
        try:
            check(orc)
        except Exception:  # an assertion or a crash both count as caught
            failed.append(check.__name__)
    assert failed, f"no pin caught mutant {mutant.__name__}"
