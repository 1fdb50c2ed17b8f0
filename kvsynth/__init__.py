"""Seeded synthetic inputs for block-sparse decode attention.

This module is shared by the tests, the benchmark and the oracle's callers.  It holds none of the
method's arithmetic (no reps, scores, selection or attention): it draws fp16 queries, keys and values,
plants "hot" blocks whose keys lean towards the query, and lays sequences out in a paged block pool.

Recipe (stands in for the long-context datasets the KTransformers article measures on):
  * q, K, V ~ N(0, 1), drawn in float32 by torch's seeded generator on the requested device and rounded
    to fp16 (round-to-nearest-even); negative zero is replaced by +0 so min/max have one answer.
  * planting: for KV head h, u_h = normalise(sum of the query heads that read h); every key row of a
    hot block gets K[t][h] += shift * u_h (shift 2.0) before rounding to fp16.
  * a seed is a 64-bit mix of (base seed, tags); each tensor, layer and chunk draws from its own seed,
    so results do not depend on how a caller chunks or orders the work.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

_MASK64 = (1 << 64) - 1


def mix_seed(*parts: int) -> int:
    """splitmix64 chain over integer tags -> a 63-bit torch seed."""
    x = 0x9E3779B97F4A7C15
    for p in parts:
        x = (x ^ (int(p) & _MASK64)) & _MASK64
        x = (x + 0x9E3779B97F4A7C15) & _MASK64
        z = x
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        x = z ^ (z >> 31)
    return x & ((1 << 63) - 1)


def _canon_fp16(x32: torch.Tensor) -> torch.Tensor:
    h = x32.to(torch.float16)
    return torch.where(h == 0, torch.zeros_like(h), h)  # -0 -> +0


def randn_fp16(shape, seed: int, device="cpu") -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return _canon_fp16(x)


def choose_blocks(seed: int, lo: int, hi: int, n: int) -> list[int]:
    """n distinct block ids from [lo, hi), seeded (CPU generator, independent of device)."""
    if hi <= lo or n <= 0:
        return []
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    perm = torch.randperm(hi - lo, generator=g)[: min(n, hi - lo)]
    return sorted(int(lo + p) for p in perm)


def query_directions(q: torch.Tensor, Hkv: int) -> torch.Tensor:
    """u_h = normalised sum of the query heads j with j // (Hq/Hkv) == h, float32 [Hkv][d]."""
    Hq, d = q.shape
    g = Hq // Hkv
    u = q.float().reshape(Hkv, g, d).sum(dim=1)
    return u / u.norm(dim=1, keepdim=True).clamp_min(1e-30)


@dataclass
class Sequence:
    """One sequence in logical order: q [Hq][d], K and V [L][Hkv][d], all fp16."""
    q: torch.Tensor
    K: torch.Tensor
    V: torch.Tensor
    hot: list = field(default_factory=list)  # hot[h] = sorted hot block ids of KV head h


def make_sequence(seed: int, L: int, Hq: int, Hkv: int, d: int = 128, B: int = 128, *,
                  hot_range=(0, 0), n_hot: int = 0, hot_per_head: bool = False,
                  shift: float = 2.0, device="cpu") -> Sequence:
    """Draw one sequence; plant ``n_hot`` hot blocks from ``hot_range`` (shared by all KV heads
    unless ``hot_per_head``)."""
    q = randn_fp16((Hq, d), mix_seed(seed, 1), device)
    K = randn_fp16((L, Hkv, d), mix_seed(seed, 2), device)
    V = randn_fp16((L, Hkv, d), mix_seed(seed, 3), device)
    hot = []
    if n_hot > 0:
        u = query_directions(q, Hkv).to(device)
        for h in range(Hkv):
            tag = h if hot_per_head else 0
            blocks = choose_blocks(mix_seed(seed, 4, tag), hot_range[0], hot_range[1], n_hot)
            hot.append(blocks)
            for b in blocks:
                rows = K[b * B:(b + 1) * B, h, :].float() + shift * u[h]
                K[b * B:(b + 1) * B, h, :] = _canon_fp16(rows)
    return Sequence(q=q, K=K, V=V, hot=hot)


@dataclass
class PagedBatch:
    """A batch laid out in a paged pool.

    k_pool, v_pool: fp16 [n_phys][Hkv][B][d]; block_table: int32 [batch][max_blocks] (logical block
    -> physical id, -1 where unused); seq_lens: int32 [batch]; q: fp16 [batch][Hq][d].
    """
    q: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    block_table: torch.Tensor
    seq_lens: torch.Tensor
    B: int

    @property
    def max_blocks(self) -> int:
        return self.block_table.shape[1]


def page_batch(seqs: list[Sequence], B: int, *, shuffle_seed: int | None = None,
               spare_blocks: int = 0, fill=float("nan"), max_blocks: int | None = None,
               device="cpu") -> PagedBatch:
    """Scatter sequences into one pool.  Physical ids are a seeded permutation when
    ``shuffle_seed`` is given (identity otherwise).  The tail of every last block and every spare
    block is filled with ``fill`` (NaN by default, so a kernel that reads past a sequence shows it)."""
    Hkv, d = seqs[0].K.shape[1], seqs[0].K.shape[2]
    nbs = [math.ceil(s.K.shape[0] / B) for s in seqs]
    n_phys = sum(nbs) + spare_blocks
    mb = max_blocks if max_blocks is not None else max(max(nbs), 1)
    if shuffle_seed is not None:
        g = torch.Generator(device="cpu")
        g.manual_seed(shuffle_seed)
        perm = torch.randperm(n_phys, generator=g)
    else:
        perm = torch.arange(n_phys)
    k_pool = torch.full((n_phys, Hkv, B, d), fill, dtype=torch.float16, device=device)
    v_pool = torch.full((n_phys, Hkv, B, d), fill, dtype=torch.float16, device=device)
    table = torch.full((len(seqs), mb), -1, dtype=torch.int32)
    nxt = 0
    for i, s in enumerate(seqs):
        L = s.K.shape[0]
        for b in range(nbs[i]):
            p = int(perm[nxt])
            nxt += 1
            table[i, b] = p
            t0, t1 = b * B, min((b + 1) * B, L)
            k_pool[p, :, : t1 - t0, :] = s.K[t0:t1].to(device).transpose(0, 1)
            v_pool[p, :, : t1 - t0, :] = s.V[t0:t1].to(device).transpose(0, 1)
    q = torch.stack([s.q for s in seqs]).to(device)
    lens = torch.tensor([s.K.shape[0] for s in seqs], dtype=torch.int32)
    return PagedBatch(q=q, k_pool=k_pool, v_pool=v_pool, block_table=table.to(device),
                      seq_lens=lens.to(device), B=B)


def pool_layer(seed: int, L: int, Hq: int, Hkv: int, d: int = 128, B: int = 128, *,
               hot_range=(0, 0), n_hot: int = 0, hot_per_head: bool = True, shift: float = 2.0,
               device="cuda", chunk_blocks: int = 256):
    """One long sequence drawn directly in pool layout (identity block table), chunk by chunk, for
    caches too large to hold twice (the 1M-token layers).  Returns (q, k_pool, v_pool, hot).

    Key/value values come from per-chunk seeds, so they differ from ``make_sequence`` for the same
    seed; a caller reads the logical cache back with ``logical_from_pool``.
    """
    nb = math.ceil(L / B)
    q = randn_fp16((Hq, d), mix_seed(seed, 1), device)
    k_pool = torch.empty((nb, Hkv, B, d), dtype=torch.float16, device=device)
    v_pool = torch.empty((nb, Hkv, B, d), dtype=torch.float16, device=device)
    for c0 in range(0, nb, chunk_blocks):
        c1 = min(nb, c0 + chunk_blocks)
        k_pool[c0:c1] = randn_fp16((c1 - c0, Hkv, B, d), mix_seed(seed, 12, c0), device)
        v_pool[c0:c1] = randn_fp16((c1 - c0, Hkv, B, d), mix_seed(seed, 13, c0), device)
    hot = []
    if n_hot > 0:
        u = query_directions(q, Hkv).to(device)
        for h in range(Hkv):
            tag = h if hot_per_head else 0
            blocks = choose_blocks(mix_seed(seed, 4, tag), hot_range[0], hot_range[1], n_hot)
            hot.append(blocks)
            if blocks:
                idx = torch.tensor(blocks, device=device)
                rows = k_pool[idx, h].float() + shift * u[h]
                k_pool[idx, h] = _canon_fp16(rows)
    tail = nb * B - L
    if tail:
        k_pool[nb - 1, :, B - tail:, :] = float("nan")
        v_pool[nb - 1, :, B - tail:, :] = float("nan")
    return q, k_pool, v_pool, hot


def logical_from_pool(pool: torch.Tensor, table_row, L: int) -> torch.Tensor:
    """Gather one sequence's [L][Hkv][d] view (on the pool's device) through its block table row."""
    B = pool.shape[2]
    nb = math.ceil(L / B)
    ids = torch.as_tensor(table_row[:nb], dtype=torch.long, device=pool.device)
    x = pool.index_select(0, ids).transpose(1, 2).reshape(nb * B, pool.shape[1], pool.shape[3])
    return x[:L]


def uniform_lengths(seed: int, n: int, lo: int, hi: int) -> list[int]:
    """n sequence lengths drawn uniformly from [lo, hi] (seeded, CPU generator)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=g)]


def pool_batch(seed: int, lens: list[int], Hq: int, Hkv: int, d: int = 128, B: int = 128, *,
               hot_ranges=None, n_hot: int = 0, shift: float = 2.0, device="cuda", chunk_blocks: int = 256):
    """A batch of sequences drawn directly into one shared paged pool (for batches too large to hold
    twice).  Sequence i owns ceil(lens[i] / B) blocks; physical ids are a seeded permutation of all
    of them.  Keys and values come from per-(sequence, chunk) seeds; the tail of each sequence's
    last block is NaN.  hot_ranges[i] = (lo, hi): n_hot planted blocks of sequence i drawn from
    [lo, hi), the same for every KV head, keys shifted by ``shift`` along the sequence's per-head
    query direction.  Returns (q [batch][Hq][d], k_pool, v_pool, block_table [batch][max_blocks]
    int32 (-1 past a sequence), hot)."""
    nbs = [math.ceil(L / B) for L in lens]
    n_phys = sum(nbs)
    mb = max(nbs)
    g = torch.Generator(device="cpu")
    g.manual_seed(mix_seed(seed, 7))
    perm = torch.randperm(n_phys, generator=g)
    table = torch.full((len(lens), mb), -1, dtype=torch.int32)
    k_pool = torch.empty((n_phys, Hkv, B, d), dtype=torch.float16, device=device)
    v_pool = torch.empty((n_phys, Hkv, B, d), dtype=torch.float16, device=device)
    qs, hot, nxt = [], [], 0
    for i, L in enumerate(lens):
        ids = perm[nxt:nxt + nbs[i]]
        nxt += nbs[i]
        table[i, : nbs[i]] = ids.to(torch.int32)
        idd = ids.to(device)
        q = randn_fp16((Hq, d), mix_seed(seed, i, 1), device)
        qs.append(q)
        for c0 in range(0, nbs[i], chunk_blocks):
            c1 = min(nbs[i], c0 + chunk_blocks)
            k_pool.index_copy_(0, idd[c0:c1], randn_fp16((c1 - c0, Hkv, B, d), mix_seed(seed, i, 12, c0), device))
            v_pool.index_copy_(0, idd[c0:c1], randn_fp16((c1 - c0, Hkv, B, d), mix_seed(seed, i, 13, c0), device))
        blocks = []
        if n_hot > 0 and hot_ranges is not None:
            u = query_directions(q, Hkv).to(device)
            blocks = choose_blocks(mix_seed(seed, i, 4), hot_ranges[i][0], hot_ranges[i][1], n_hot)
            if blocks:
                pid = idd[torch.tensor(blocks, device=device)]
                rows = k_pool[pid].float() + shift * u[None, :, None, :]
                k_pool[pid] = _canon_fp16(rows)
        hot.append(blocks)
        tail = nbs[i] * B - L
        if tail:
            k_pool[int(ids[-1]), :, B - tail:, :] = float("nan")
            v_pool[int(ids[-1]), :, B - tail:, :] = float("nan")
    return torch.stack(qs), k_pool, v_pool, table.to(device), hot
