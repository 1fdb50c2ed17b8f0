"""Plain, slow fp64 CPU oracle for block-sparse long-context decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run this module: only the
tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no
code, header, table or helper with the HIP library; the two meet only through the seeded inputs.

What it computes follows the KTransformers long-context sparse-attention article
("KTransformers 长上下文稀疏注意力实战", lmnt.cn), whose sections are cited per function as
[KT-LC §n]:
  * §4.2  the cache is split into Initial (head, always attended), Context (middle, retrieved
          sparsely) and Local (tail, always attended);
  * §4.3  Context is cut into fixed-size blocks; each block gets representative ("rep") keys by one of
          Max (channel-wise max), Mean (channel-wise mean), Quest (channel-wise min and max, two
          reps), Fix (tokens at a fixed interval) -- Dynamic needs prefill attention scores and is
          not part of this oracle;
  * §3.1  Quest's block score: per channel the larger of q*kmax and q*kmin, summed over channels --
          an upper bound on q.k for every key of the block;
  * §4.3  other reps are scored by their similarity with the query (the InfLLM equation the article
          refers to is not printed; reading R7 below);
  * §4.5  head_select_mode SEPARATE (each KV head selects for itself under GQA) or SHARED (all KV
          heads select jointly); top ``second_block_count`` blocks are selected;
  * §4.6  after selection, ordinary attention runs over the retrieved cache; the pseudocode scales
          logits by 1/sqrt(head_dim).

  * the operator's configuration lists kv_type among FP16, FP32, Q4_0 and Q8_0 cache precisions
    (the article's config list; the instagit page's operator constructor).  Q8_0 is the llama.cpp
    block format the pages name but do not define; see R22.

Readings taken where the pages are silent (each is the spec here):
  R1  Initial and Local are rounded outward to whole blocks: I_b = B*ceil(I/B),
      L_loc = max(I_b, B*floor((L-W)/B)); candidates are the full blocks in [I_b, L_loc).
      If L <= I_b everything is Initial.
  R3  top-k counts Context blocks only; k_eff = min(k, n_cand) (R4).
  R5  block scores carry no softmax scale.
  R7  a multi-rep block (Fix) scores sum over reps of q.rep (parity unpinned by the pages).
  R8  Fix reps are the block's tokens at offsets r*(B/rep_num), r = 0..rep_num-1.
  R10 query head j reads KV head j // (Hq/Hkv).
  R11 SEPARATE group score = sum over the query heads of the group (parity unpinned by the pages).
  R12 ties in top-k go to the lower block index; the selection is reported in ascending order.
  R14 attention: softmax of q.k/sqrt(d) over the attended tokens only.
  R23 Dynamic reps (the article's fifth rep method: each token's cumulative attention score, the
      top tokens of each block become its reps).  The article leaves the scoring method open; here
      a token's score is the attention it receives from the n_obs observation queries -- the last
      n_obs tokens of the prompt, at positions L-n_obs .. L-1, each attending causally (keys at
      positions <= its own) with scale 1/sqrt(d) -- summed over those queries and over the query
      heads of the selection group (SEPARATE: the g heads of a KV head; SHARED: all heads).  A
      block's reps are the K rows of its rep_num highest-scoring tokens (ties to the lower token),
      in ascending token order, and a Dynamic block is scored like Fix (sum over reps of q.rep).
  R24 Preselect (the article's optional module after SnapKV: before decoding, blocks are chosen by
      the attention the question's tokens pay the context; later selections are confined to them).
      A block's preselect score is the sum of its tokens' scores (R23's token scores); the
      preselect_block_count best candidates (ties to the lower block) form the set; a decode step
      then ranks only the current candidates inside the set, k_eff = min(k, their number) -- so
      with k >= the set's size the set itself is attended.
  R26 Pooled preselect (the article's framework pseudocode, §4.6 preselect_block: the window's
      votes are pooled by pool1d with padding kernel_size // 2 and stride 1, the best tokens are
      taken, and the set is the blocks they fall in).  The pages contradict themselves here: §4.5
      says block size 1 with preselect on is SnapKV without pooling, the pseudocode pools.  Both
      are offered: pool_kernel = 0 is R24; an odd pool_kernel >= 1 is this reading.  The vote is
      restricted to the Context tokens (the pseudocode slices Initial and Local off before
      pooling), pooled by an average over pool_kernel tokens centred on each token with zeros
      beyond the Context (torch's avg_pool1d with count_include_pad), and tokens are taken in
      descending pooled vote (ties to the lower token) until preselect_block_count distinct blocks
      are hit.  That is the same as ranking each candidate block by its best pooled token (ties to
      the lower block), which is how it is computed.  The pooling kind is not named; the average
      is SnapKV's usual choice.
  R25 kv_type Q4_0 (llama.cpp's other block format the list names, restated): per 32 channels of a
      token's row, m = the value of largest magnitude (the first one on ties), d = m / -8,
      codes q = min(15, trunc(x * (1/d) + 8.5)) in 0..15, all fp32; d stored as fp16; the cached
      value is fp16(d) * (q - 8).  An all-zero block has d = 0 and codes 8.
  R27 kv_type INT8 per token and head (the int8 cache with one dynamic scale per token and head
      of the page "Long context: 262k with KVarN, and the built-in KV modes", section "The built-in
      per-token-head modes"; it names the granularity and the fp32 scale, not the arithmetic, which
      is read as Q8_0's): per token's K or V row of one KV head,
      s = max|x| / 127 in fp32, stored as fp32; codes round(x * (1/s)), ties away from zero, all
      fp32 operations; an all-zero row has s = 0 and codes 0.  The cached value is the fp32
      product s * code.
  R28 kv_type INT4 per token and head (the page's int4 per-token-head cache: a dynamic scale per
      token and head, with a rotation and asymmetric zero-points, neither defined there).  Read as
      the usual asymmetric integer quantization with a zero point, without a rotation: per token's
      K or V row of one KV head, lo = min(0, min x), hi = max(0, max x) (the range holds 0, so 0 is
      cached exactly), s = (hi - lo) / 15, inv = 1 / s, the zero point z = rint(-lo * inv) clamped
      to 0..15 and codes q = clamp(rint(x * inv) + z, 0, 15), rint rounding half to even; every
      step an fp32 operation; s stored as fp32, z as a byte.  An all-zero row has s = 0, z = 0 and
      codes 0.  The cached value is the fp32 product s * (q - z).  Parity unpinned by the pages:
      the pins hold this reading.
  R22 kv_type Q8_0 (the published llama.cpp format, restated): every run of 32 consecutive channels
      of one token's key or value row is a block with scale d = max|x| / 127 and codes
      q = round(x / d) (ties away from zero), d stored as fp16; the cached value is fp16(d) * q.
      d, 1/d and x * (1/d) are fp32 operations (so the codes are the ones an fp32 implementation
      takes); an all-zero block has d = 0 and codes 0.  Reps of a Q8_0 cache are taken over the
      cached (dequantized) keys and stored as fp16 (Mean: fp32), and attention runs over the
      dequantized keys and values.
Pins (tests/test_oracle_pins.py, tests/test_oracle_bruteforce.py): Quest upper-bound invariant in
exact integer arithmetic; dense/masked attention against torch's scaled_dot_product_attention in
float64; brute force with Fractions and rank-by-counting top-k on tiny caches; closed forms for Mean
and Fix; SHARED = sum of SEPARATE; softmax identities.  R7 and R11 stay "parity unpinned" by the
pages: the readings themselves are what the GPU is held to.

All arithmetic is float64 after an exact widening of the fp16 inputs.
"""
from __future__ import annotations

import math

import numpy as np

QUEST, MAX, MEAN, FIX = "quest", "max", "mean", "fix"
SEPARATE, SHARED = "separate", "shared"
REP_METHODS = (QUEST, MAX, MEAN, FIX)


# ----------------------------------------------------------------------------------------------
# O1. Regions  [KT-LC §4.2 Initial / Context / Local; §4.3 fixed-size Context blocks]
# ----------------------------------------------------------------------------------------------
def regions(L: int, B: int, initial_len: int, local_len: int):
    """Split a cache of L tokens into Initial / Context candidates / Local (reading R1).

    Returns (init_end, local_start, candidates): Initial = [0, init_end), Local = [local_start, L),
    candidates = list of logical block ids b whose tokens [b*B, (b+1)*B) form the Context.
    """
    I_b = B * math.ceil(initial_len / B)
    if L <= I_b:
        return L, L, []
    L_loc = max(I_b, B * math.floor((L - local_len) / B))
    return I_b, L_loc, list(range(I_b // B, L_loc // B))


# ----------------------------------------------------------------------------------------------
# O2. Block reps  [KT-LC §4.3 table of rep methods; §3.1 Quest "Reduced Keys"]
# ----------------------------------------------------------------------------------------------
def rep_count(method: str, rep_num: int) -> int:
    """Reps per (block, KV head): Quest keeps a min and a max key (fixed at 2, §4.3), Max and Mean
    one, Fix ``rep_num``."""
    if method == QUEST:
        return 2
    if method in (MAX, MEAN):
        return 1
    if method == FIX:
        return rep_num
    raise ValueError(method)


def block_reps(K, B: int, method: str, rep_num: int = 1, blocks=None):
    """Reps of full blocks of one sequence's keys.

    K: [L][Hkv][d] (fp16 or any float), logical token order.
    blocks: logical block ids to build (default: every full block, b < L // B).
    Returns float64 array [len(blocks)][Hkv][R][d]; Quest puts the min key at r=0, max key at r=1.
    """
    L, Hkv, d = K.shape
    if blocks is None:
        blocks = range(L // B)
    blocks = list(blocks)
    R = rep_count(method, rep_num)
    out = np.empty((len(blocks), Hkv, R, d), dtype=np.float64)
    for i, b in enumerate(blocks):
        assert (b + 1) * B <= L, "reps are defined for full blocks only"
        tile = np.asarray(K[b * B:(b + 1) * B], dtype=np.float64)  # [B][Hkv][d]
        if method == QUEST:
            out[i, :, 0, :] = tile.min(axis=0)
            out[i, :, 1, :] = tile.max(axis=0)
        elif method == MAX:
            out[i, :, 0, :] = tile.max(axis=0)
        elif method == MEAN:
            out[i, :, 0, :] = tile.sum(axis=0) / B
        elif method == FIX:
            assert B % rep_num == 0, "Fix needs rep_num | block_size"
            stride = B // rep_num
            for r in range(rep_num):
                out[i, :, r, :] = tile[r * stride]
        else:
            raise ValueError(method)
    return out


# ----------------------------------------------------------------------------------------------
# O3. Per-head block scores  [KT-LC §3.1 Quest bound; §4.3 rep similarity]
# ----------------------------------------------------------------------------------------------
def head_scores(q, reps, method: str):
    """s[i][j] = score of block i for query head j (no softmax scale, reading R5).

    q: [Hq][d]; reps: [nblk][Hkv][R][d] from ``block_reps``.
    Quest: sum_c max(q_c*kmax_c, q_c*kmin_c).  Max / Mean / Fix: sum_r q.rep_r (R7).
    """
    q = np.asarray(q, dtype=np.float64)
    Hq, d = q.shape
    nblk, Hkv, R, _ = reps.shape
    g = Hq // Hkv
    s = np.empty((nblk, Hq), dtype=np.float64)
    for j in range(Hq):
        h = j // g  # R10: contiguous GQA groups
        if method == QUEST:
            kmin, kmax = reps[:, h, 0, :], reps[:, h, 1, :]
            s[:, j] = np.maximum(q[j] * kmax, q[j] * kmin).sum(axis=1)
        else:
            s[:, j] = (reps[:, h, :, :] * q[j]).sum(axis=(1, 2))
    return s


# ----------------------------------------------------------------------------------------------
# O4. Group scores  [KT-LC §4.5 head_select_mode]
# ----------------------------------------------------------------------------------------------
def group_scores(s, Hkv: int, mode: str):
    """SEPARATE: one score row per KV head, summed over its query heads (R11).
    SHARED: a single row, summed over all query heads.  Returns [G][nblk]."""
    nblk, Hq = s.shape
    g = Hq // Hkv
    if mode == SEPARATE:
        return np.stack([s[:, h * g:(h + 1) * g].sum(axis=1) for h in range(Hkv)])
    if mode == SHARED:
        return s.sum(axis=1)[None, :]
    raise ValueError(mode)


# ----------------------------------------------------------------------------------------------
# O5. Top-k  [KT-LC §3.1 "select top-k blocks"; §4.5 second_block_count]
# ----------------------------------------------------------------------------------------------
def select_topk(scores_row, cand, k: int):
    """The k_eff = min(k, len(cand)) best candidates by (score desc, block asc), ascending order."""
    ranked = sorted(range(len(cand)), key=lambda i: (-scores_row[i], cand[i]))
    return sorted(cand[i] for i in ranked[:min(k, len(cand))])


# ----------------------------------------------------------------------------------------------
# O6. Exact attention over the retrieved cache  [KT-LC §4.6 attn(query, kvcache_after_retrieval)]
# ----------------------------------------------------------------------------------------------
def attended_tokens(L: int, B: int, init_end: int, local_start: int, sel):
    """Initial tokens, then every token of each selected block, then Local tokens."""
    toks = list(range(0, min(init_end, L)))
    for b in sel:
        toks.extend(range(b * B, (b + 1) * B))
    toks.extend(range(local_start, L))
    return toks


def attention(q, K, V, tokens_per_head, scale=None):
    """o_j = softmax_t(q_j.K[t]*scale) @ V[t] over t in tokens_per_head[j]; float64 [Hq][d]."""
    q = np.asarray(q, dtype=np.float64)
    Hq, d = q.shape
    Hkv = K.shape[1]
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.empty((Hq, d), dtype=np.float64)
    for j in range(Hq):
        h = j // g
        T = np.asarray(tokens_per_head[j], dtype=np.int64)
        Kt = np.asarray(K[T, h, :], dtype=np.float64)
        Vt = np.asarray(V[T, h, :], dtype=np.float64)
        z = (Kt @ q[j]) * scale
        w = np.exp(z - z.max())
        out[j] = (w @ Vt) / w.sum()
    return out


# ----------------------------------------------------------------------------------------------
# The whole decode step for one sequence  [KT-LC §4.6: retrieval_kvcache then attn]
# ----------------------------------------------------------------------------------------------
def decode_step(q, K, V, *, B, initial_len, local_len, topk, method, rep_num=1,
                mode=SEPARATE, scale=None, reps=None):
    """One decode step for one sequence whose cache (current token included) is K, V [L][Hkv][d].

    Returns a dict with regions, candidate ids, reps of the candidates, per-head and group scores,
    the selection per group (ascending), attended token lists per query head and the fp64 output.
    ``reps`` may be passed in (from ``block_reps`` over the candidates) to skip rebuilding them.
    """
    L, Hkv, d = K.shape
    Hq = q.shape[0]
    g = Hq // Hkv
    init_end, local_start, cand = regions(L, B, initial_len, local_len)
    if reps is None:
        reps = block_reps(K, B, method, rep_num, blocks=cand)
    s = head_scores(q, reps, method) if cand else np.zeros((0, Hq))
    S = group_scores(s, Hkv, mode) if cand else np.zeros((Hkv if mode == SEPARATE else 1, 0))
    sel = [select_topk(S[gi], cand, topk) for gi in range(S.shape[0])]
    toks = []
    for j in range(Hq):
        gi = (j // g) if mode == SEPARATE else 0
        toks.append(attended_tokens(L, B, init_end, local_start, sel[gi]))
    out = attention(q, K, V, toks, scale)
    return dict(init_end=init_end, local_start=local_start, cand=cand, reps=reps,
                head_scores=s, scores=S, sel=sel, tokens=toks, out=out)


# ----------------------------------------------------------------------------------------------
# O7. Q8_0 cache precision  [the configuration's kv_type: FP16 / FP32 / Q4_0 / Q8_0; reading R22]
# ----------------------------------------------------------------------------------------------
Q8_GROUP = 32


def quantize_q8_0(x):
    """Codes and scales of x [..., d] (d a multiple of 32) in the Q8_0 format (reading R22).

    Returns (codes int8 [..., d], scales float16 [..., d // 32]).  The scale, its reciprocal and the
    scaled values are fp32 operations; the rounding to a code is ties-away-from-zero.
    """
    x = np.asarray(x, dtype=np.float32)
    *lead, d = x.shape
    assert d % Q8_GROUP == 0
    xg = x.reshape(*lead, d // Q8_GROUP, Q8_GROUP)
    amax = np.abs(xg).max(axis=-1)                                  # fp32, exact
    dsc = (amax / np.float32(127.0)).astype(np.float32)             # fp32 division
    with np.errstate(divide="ignore"):
        inv = np.where(dsc != 0, np.float32(1.0) / dsc, np.float32(0.0)).astype(np.float32)
    v = (xg * inv[..., None]).astype(np.float32)                    # fp32 product
    v64 = v.astype(np.float64)
    codes = (np.sign(v64) * np.floor(np.abs(v64) + 0.5)).astype(np.int8)  # ties away from zero
    return codes.reshape(*lead, d), dsc.astype(np.float16)


def dequantize_q8_0(codes, scales):
    """The cached values fp16(d) * q as float64 [..., d] (exact: 11-bit scale times 8-bit code)."""
    codes = np.asarray(codes, dtype=np.int8)
    *lead, d = codes.shape
    sc = np.asarray(scales, dtype=np.float16).astype(np.float64)
    cg = codes.astype(np.float64).reshape(*lead, d // Q8_GROUP, Q8_GROUP)
    return (cg * sc[..., None]).reshape(*lead, d)


def quantize_int8_pth(x):
    """Codes (int8 [..., d]) and fp32 scales ([...]) of x [..., d], one scale per row (reading
    R27).  The scale, its reciprocal and the scaled values are fp32 operations; codes round ties
    away from zero."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)                                   # fp32, exact
    s = (amax / np.float32(127.0)).astype(np.float32)               # fp32 division
    with np.errstate(divide="ignore"):
        inv = np.where(s != 0, np.float32(1.0) / np.where(s != 0, s, 1), np.float32(0.0)).astype(np.float32)
    v = (x * inv[..., None]).astype(np.float32).astype(np.float64)  # fp32 product
    codes = (np.sign(v) * np.floor(np.abs(v) + 0.5)).astype(np.int8)
    return codes, s


def dequantize_int8_pth(codes, scales):
    """The cached values fp32(s * q) as float64 [..., d] (reading R27)."""
    c = np.asarray(codes, dtype=np.int8).astype(np.float32)
    sc = np.asarray(scales, dtype=np.float32)
    return (c * sc[..., None]).astype(np.float32).astype(np.float64)


def quantize_int4_pth(x):
    """Codes (uint8 0..15 [..., d]), fp32 scales ([...]) and zero points (uint8 [...]) of x [..., d],
    one scale and zero point per row (reading R28).  Range, scale, reciprocal and scaled values are
    fp32 operations; rint rounds half to even."""
    x = np.asarray(x, dtype=np.float32)
    lo = np.minimum(x.min(axis=-1), np.float32(0.0)).astype(np.float32)   # the range holds 0
    hi = np.maximum(x.max(axis=-1), np.float32(0.0)).astype(np.float32)
    s = ((hi - lo).astype(np.float32) / np.float32(15.0)).astype(np.float32)  # fp32 ops
    nz = s != 0
    with np.errstate(divide="ignore"):
        inv = np.where(nz, np.float32(1.0) / np.where(nz, s, 1), np.float32(0.0)).astype(np.float32)
    z = np.clip(np.rint((-lo * inv).astype(np.float32).astype(np.float64)), 0, 15)
    z = np.where(nz, z, 0).astype(np.int64)
    t = np.rint((x * inv[..., None]).astype(np.float32).astype(np.float64)).astype(np.int64)
    codes = np.clip(t + z[..., None], 0, 15).astype(np.uint8)
    return codes, s, z.astype(np.uint8)


def dequantize_int4_pth(codes, scales, zeros):
    """The cached values fp32(s * (q - z)) as float64 [..., d] (reading R28)."""
    c = np.asarray(codes, dtype=np.int64) - np.asarray(zeros, dtype=np.int64)[..., None]
    sc = np.asarray(scales, dtype=np.float32)
    return (c.astype(np.float32) * sc[..., None]).astype(np.float32).astype(np.float64)


def quantize_q4_0(x):
    """Codes (uint8 0..15) and fp16 scales of x [..., d] in the Q4_0 format (reading R25)."""
    x = np.asarray(x, dtype=np.float32)
    *lead, d = x.shape
    assert d % Q8_GROUP == 0
    xg = x.reshape(*lead, d // Q8_GROUP, Q8_GROUP)
    first = np.abs(xg).argmax(axis=-1)                              # first index of the largest |x|
    m = np.take_along_axis(xg, first[..., None], -1)[..., 0]
    m = np.where(np.abs(xg).max(axis=-1) > 0, m, np.float32(0.0)).astype(np.float32)  # +0 if all zero
    dsc = (m / np.float32(-8.0)).astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(dsc != 0, np.float32(1.0) / np.where(dsc != 0, dsc, 1), np.float32(0.0)).astype(np.float32)
    v = ((xg * inv[..., None]).astype(np.float32) + np.float32(8.5)).astype(np.float32)
    codes = np.minimum(15, np.trunc(v.astype(np.float64))).astype(np.uint8)
    return codes.reshape(*lead, d), dsc.astype(np.float16)


def dequantize_q4_0(codes, scales):
    """The cached values fp16(d) * (q - 8) as float64 [..., d]."""
    codes = np.asarray(codes, dtype=np.int64)
    *lead, d = codes.shape
    sc = np.asarray(scales, dtype=np.float16).astype(np.float64)
    cg = (codes - 8).astype(np.float64).reshape(*lead, d // Q8_GROUP, Q8_GROUP)
    return (cg * sc[..., None]).reshape(*lead, d)


def stored_reps(reps, method: str):
    """Reps as the rep pool holds them when they are not copies of fp16 keys (a quantized cache): fp16
    with round-to-nearest-even, Mean fp32 (reading R22)."""
    reps = np.asarray(reps, dtype=np.float64)
    if method == MEAN:
        return reps.astype(np.float32).astype(np.float64)
    return reps.astype(np.float16).astype(np.float64)


# ----------------------------------------------------------------------------------------------
# O8. Dynamic reps  [KT-LC §4.3 rep table: Dynamic, the block's tokens with the highest cumulative
#     attention score; reading R23]
# ----------------------------------------------------------------------------------------------
def token_importance(q_obs, K, mode: str, scale=None):
    """Cumulative attention score of every cached token (reading R23).

    q_obs: [n_obs][Hq][d], the queries of the last n_obs tokens of the cache (positions L-n_obs ..
    L-1); K: [L][Hkv][d].  Returns float64 [G][L] with G = Hkv (SEPARATE) or 1 (SHARED): the sum,
    over observation queries i and the group's query heads j, of softmax_t(scale * q_ij . K[t]) over
    t <= L - n_obs + i (zero beyond).
    """
    q_obs = np.asarray(q_obs, dtype=np.float64)
    n_obs, Hq, d = q_obs.shape
    L, Hkv, _ = K.shape
    assert 1 <= n_obs <= L
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    imp = np.zeros((Hkv, L))
    for h in range(Hkv):
        Kh = np.asarray(K[:, h, :], dtype=np.float64)
        for i in range(n_obs):
            p = L - n_obs + i  # position of observation query i
            for j in range(h * g, (h + 1) * g):
                z = (Kh[: p + 1] @ q_obs[i, j]) * scale
                w = np.exp(z - z.max())
                imp[h, : p + 1] += w / w.sum()
    if mode == SEPARATE:
        return imp
    if mode == SHARED:
        return imp.sum(axis=0, keepdims=True)
    raise ValueError(mode)


def dynamic_reps(K, imp, B: int, rep_num: int, mode: str, blocks):
    """Reps of full blocks (reading R23): per block and KV head, the K rows of the rep_num tokens
    with the largest importance (ties to the lower token), in ascending token order.

    K: [L][Hkv][d]; imp: [G][L] from ``token_importance``.  Returns float64 [len(blocks)][Hkv][rep_num][d]
    and the chosen token offsets [len(blocks)][Hkv][rep_num].
    """
    L, Hkv, d = K.shape
    blocks = list(blocks)
    out = np.empty((len(blocks), Hkv, rep_num, d))
    picked = np.empty((len(blocks), Hkv, rep_num), dtype=np.int64)
    for n, b in enumerate(blocks):
        assert (b + 1) * B <= L, "reps are defined for full blocks only"
        for h in range(Hkv):
            row = imp[h if mode == SEPARATE else 0, b * B:(b + 1) * B]
            order = sorted(range(B), key=lambda t: (-row[t], t))[:rep_num]
            toks = sorted(order)
            picked[n, h] = toks
            out[n, h] = np.asarray(K[[b * B + t for t in toks], h, :], dtype=np.float64)
    return out, picked


# ----------------------------------------------------------------------------------------------
# O9. Preselect  [KT-LC §4.4 Preselect (after SnapKV); §4.5 preselect_block_count; §4.6
#     preselect_block; readings R24, R26]
# ----------------------------------------------------------------------------------------------
def pooled_votes(row, lo: int, hi: int, pool_kernel: int):
    """Reading R26: the votes of the Context tokens [lo, hi), each averaged with its pool_kernel // 2
    neighbours on either side; tokens outside [lo, hi) count as zero, the divisor is always
    pool_kernel.  Returns float64 [hi - lo]."""
    h = pool_kernel // 2
    out = np.zeros(hi - lo)
    for t in range(lo, hi):
        acc = 0.0
        for u in range(t - h, t + h + 1):
            if lo <= u < hi:
                acc += row[u]
        out[t - lo] = acc / pool_kernel
    return out


def preselect_scores(imp, L: int, B: int, initial_len: int, local_len: int, pool_kernel: int = 0):
    """Per group, the preselect score of each candidate block: the sum of its tokens' scores
    (pool_kernel = 0, reading R24) or its best pooled vote (odd pool_kernel, reading R26).
    Returns (scores [G][n_cand], candidates)."""
    lo, hi, cand = regions(L, B, initial_len, local_len)
    rows = []
    for row in np.asarray(imp, dtype=np.float64):
        if pool_kernel == 0:
            rows.append([row[b * B:(b + 1) * B].sum() for b in cand])
        else:
            pv = pooled_votes(row, lo, hi, pool_kernel) if cand else np.zeros(0)
            rows.append([pv[b * B - lo:(b + 1) * B - lo].max() for b in cand])
    return rows, cand


def preselect_blocks(imp, L: int, B: int, initial_len: int, local_len: int, n_presel: int,
                     pool_kernel: int = 0):
    """Per group: the n_presel candidate blocks with the best preselect score (``preselect_scores``;
    ties to the lower block), ascending.  imp: [G][L] token scores (``token_importance``)."""
    rows, cand = preselect_scores(imp, L, B, initial_len, local_len, pool_kernel)
    return [select_topk(bs, cand, n_presel) for bs in rows]


def decode_step_preselected(q, K, V, presel, *, B, initial_len, local_len, topk, method, rep_num=1,
                            mode=SEPARATE, scale=None, reps=None):
    """``decode_step`` with each group's selection confined to its preselected blocks that are still
    candidates (reading R24).  presel: per group, ascending block ids."""
    r = decode_step(q, K, V, B=B, initial_len=initial_len, local_len=local_len, topk=0,
                    method=method, rep_num=rep_num, mode=mode, scale=scale, reps=reps)
    cand = r["cand"]
    L, Hkv, d = K.shape
    g = q.shape[0] // Hkv
    pos = {b: i for i, b in enumerate(cand)}
    sel = []
    for gi, ps in enumerate(presel):
        allowed = [b for b in ps if b in pos]
        row = [r["scores"][gi][pos[b]] for b in allowed]
        sel.append(select_topk(row, allowed, topk))
    toks = []
    for j in range(q.shape[0]):
        gi = (j // g) if mode == SEPARATE else 0
        toks.append(attended_tokens(L, B, r["init_end"], r["local_start"], sel[gi]))
    r.update(sel=sel, tokens=toks, out=attention(q, K, V, toks, scale))
    return r
