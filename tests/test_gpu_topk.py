"""Top-k block selection on crafted score rows (needs an MI355X).

The score rows are drawn directly, so the selection kernels meet what model data rarely gives them:
whole rows of equal scores, a handful of distinct values (every histogram bin crowded), +0 mixed
with -0, and candidate counts on both sides of every size at which the kernels change strategy
(keys held in registers at 4, 8, 16 or 32 per lane, keys staged in LDS, keys re-read).  The
expected selection is the oracle's: the k best by score, ties to the lower block index, ascending.
"""
from __future__ import annotations

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

DEV = "cuda"
B = 128
PATTERNS = ("randn", "int8values", "const", "two", "signed_zero")


def score_row(pattern: str, n: int, seed: int) -> np.ndarray:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    if pattern == "randn":
        x = torch.randn(n, generator=g)
    elif pattern == "int8values":  # few distinct values: every bin that is used is crowded
        x = torch.randint(0, 8, (n,), generator=g).float()
    elif pattern == "const":
        x = torch.full((n,), 3.25)
    elif pattern == "two":  # mostly one value, a few larger ones
        x = torch.where(torch.rand(n, generator=g) < 0.02, 2.0, -1.5)
    else:  # +0 and -0 (one key), and some positive and negative values
        r = torch.rand(n, generator=g)
        x = torch.where(r < 0.45, torch.tensor(0.0), torch.tensor(-0.0))
        x = torch.where(r > 0.97, torch.randn(n, generator=g).abs() + 1.0, x)
        x = torch.where((r > 0.9) & (r <= 0.97), -torch.randn(n, generator=g).abs() - 1.0, x)
    return x.float().numpy()


def run_rows(n: int, k: int, seed: int):
    c = kvs.Config(num_q_heads=1, num_kv_heads=1, initial_len=0, local_len=0, topk=k,
                   rep_method="max", head_select_mode="separate")
    rows = [score_row(p, n, kvsynth.mix_seed(seed, i)) for i, p in enumerate(PATTERNS)]
    scores = torch.tensor(np.stack(rows)[:, None, :], dtype=torch.float32, device=DEV)
    lens = torch.full((len(rows),), n * B, dtype=torch.int32, device=DEV)
    sel, cnt = ops.topk_blocks(c, scores, lens)
    torch.cuda.synchronize()
    sel, cnt = sel.cpu(), cnt.cpu()
    cand = list(range(n))
    for i, p in enumerate(PATTERNS):
        ref = orc.select_topk(rows[i], cand, k)
        k_eff = len(ref)
        got = sel[i, 0].tolist()
        assert int(cnt[i, 0]) == k_eff, (p, n, k, int(cnt[i, 0]))
        assert got[:k_eff] == ref, (p, n, k, "first differences",
                                    [(a, b) for a, b in zip(got, ref) if a != b][:5])
        assert all(x == -1 for x in got[k_eff:]), (p, n, k, "padding")


# candidate counts around each change of strategy of the 1024-lane selection kernel
N_VALUES = [1, 2, 63, 64, 65, 1000, 4096, 4097, 8192, 8193, 16384, 16385, 40000]


@pytest.mark.parametrize("n", N_VALUES)
def test_topk_crafted_rows(n):
    print(f"[case] topk crafted rows n={n}", flush=True)
    for j, k in enumerate(sorted({1, 7, 64, 96, 97, max(1, n // 2), max(1, n - 1), n, n + 5})):
        run_rows(n, k, kvsynth.mix_seed(101, n, j))


def identical_block_pool(nb: int, Hkv: int, seed: int):
    blkK = kvsynth.randn_fp16((1, Hkv, B, 128), kvsynth.mix_seed(seed, 1), DEV)
    blkV = kvsynth.randn_fp16((1, Hkv, B, 128), kvsynth.mix_seed(seed, 2), DEV)
    return blkK, blkV, blkK.expand(nb, -1, -1, -1).contiguous(), blkV.expand(nb, -1, -1, -1).contiguous()


# number of blocks, so that the candidates sit in each size class of the fused step's selection
@pytest.mark.parametrize("nb", [900, 1500, 3000, 6000, 9000])
def test_step_all_blocks_equal(nb):
    """Every block is a copy of one block, so every candidate scores the same (bitwise: same inputs,
    same arithmetic): the fused step must take the first k candidates, and attend exactly them."""
    print(f"[case] fused step, {nb} identical blocks", flush=True)
    Hq, Hkv, I, W, k = 4, 1, 128, 256, 64
    c = kvs.Config(num_q_heads=Hq, num_kv_heads=Hkv, initial_len=I, local_len=W, topk=k,
                   rep_method="quest", head_select_mode="separate")
    blkK, blkV, k_pool, v_pool = identical_block_pool(nb, Hkv, kvsynth.mix_seed(202, nb))
    q = kvsynth.randn_fp16((1, Hq, 128), kvsynth.mix_seed(202, nb, 3), DEV)
    table = torch.arange(nb, dtype=torch.int32, device=DEV)[None]
    L = nb * B
    lens = torch.tensor([L], dtype=torch.int32, device=DEV)
    rp = ops.alloc_rep_pool(c, nb, DEV)
    ops.build_reps(c, k_pool, torch.arange(nb, dtype=torch.int32), rp)
    out, sel, cnt = ops.decode_step(c, q, k_pool, v_pool, rp, table, lens)
    torch.cuda.synchronize()
    init_end, local_start, cand = orc.regions(L, B, I, W)
    ref_sel = orc.select_topk(np.zeros(len(cand)), cand, k)
    assert ref_sel == cand[:k]
    assert int(cnt[0, 0]) == k and sel[0, 0].tolist() == ref_sel, sel[0, 0].tolist()[:10]
    toks = orc.attended_tokens(L, B, init_end, local_start, ref_sel)
    pos = np.asarray(toks) % B
    Kb = blkK[0].transpose(0, 1).cpu().numpy()  # [B][Hkv][d]
    Vb = blkV[0].transpose(0, 1).cpu().numpy()
    ref = orc.attention(q[0].cpu().numpy(), Kb[pos], Vb[pos], [list(range(len(toks)))] * Hq)
    err = float(np.abs(out[0].double().cpu().numpy() - ref).max())
    assert err <= 2e-3, err


@pytest.mark.parametrize("n", [1000, 4097, 8192])
def test_topk_nonfinite_rows_stay_well_formed(n):
    """NaN and infinite scores are outside the contract (their ranking is unspecified), but the
    output must stay well formed: k_eff entries, distinct candidate ids in ascending order, the rest
    -1.  Rows with a few NaNs, with +-inf, and with NaN only."""
    print(f"[case] topk non-finite rows n={n}", flush=True)
    k = 64
    c = kvs.Config(num_q_heads=1, num_kv_heads=1, initial_len=0, local_len=0, topk=k,
                   rep_method="max", head_select_mode="separate")
    g = torch.Generator(device="cpu")
    g.manual_seed(kvsynth.mix_seed(303, n))
    base = torch.randn(4, n, generator=g)
    base[0, torch.randint(0, n, (17,), generator=g)] = float("nan")
    base[1, torch.randint(0, n, (9,), generator=g)] = float("inf")
    base[1, torch.randint(0, n, (9,), generator=g)] = float("-inf")
    base[2, :] = float("nan")
    base[3, torch.randint(0, n, (5,), generator=g)] = -float("nan")
    scores = base[:, None, :].float().to(DEV)
    lens = torch.full((4,), n * B, dtype=torch.int32, device=DEV)
    sel, cnt = ops.topk_blocks(c, scores, lens)
    torch.cuda.synchronize()
    sel, cnt = sel.cpu(), cnt.cpu()
    for i in range(4):
        got = sel[i, 0].tolist()
        assert int(cnt[i, 0]) == k, (i, int(cnt[i, 0]))
        assert all(0 <= x < n for x in got[:k]), (i, got[:k])
        assert all(a < b for a, b in zip(got[:k], got[1:k])), (i, "not ascending / distinct")
        assert all(x == -1 for x in got[k:]), (i, "padding")
