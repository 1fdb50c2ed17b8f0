"""kvs_decode_step_noalloc (needs an MI355X): the decode step with its workspace in the library's
static device scratch, for callers that cannot allocate.  Called through the C ABI twice in a row --
a larger input, then a smaller one, so the second call finds the first call's contents in the
scratch -- and each result checked against kvs_decode_step on the same inputs with a workspace of
its own: selections and counts equal, outputs within the attention tolerance of the parity tests
(2e-3; the two run the same kernels, so they are expected to be bit-equal)."""
from __future__ import annotations

import sys

import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("no GPU", allow_module_level=True)

import block_sparse_kv_amd as kvs  # noqa: E402
from block_sparse_kv_amd import binding as Bd  # noqa: E402
from block_sparse_kv_amd import ops  # noqa: E402

import kvsynth  # noqa: E402

DEV = "cuda"
B = 128
ATOL = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _case(seed, lens, mode, rep, k):
    c = kvs.Config(num_q_heads=32, num_kv_heads=8, initial_len=128, local_len=2048, topk=k,
                   rep_method=rep, head_select_mode=mode)
    seqs = [kvsynth.make_sequence(kvsynth.mix_seed(seed, i), L, 32, 8, hot_range=(1, L // B - 20), n_hot=6,
                                  device=DEV) for i, L in enumerate(lens)]
    pb = kvsynth.page_batch(seqs, B, shuffle_seed=seed, spare_blocks=2, device=DEV)
    rp = ops.alloc_rep_pool(c, pb.k_pool.shape[0], DEV)
    ids = torch.cat([pb.block_table[i, : L // B] for i, L in enumerate(lens)]).cpu()
    ops.build_reps(c, pb.k_pool, ids, rp)
    return c, pb, rp


def _noalloc(c, pb, rp):
    batch, mb = pb.block_table.shape
    out = torch.empty((batch, 32, 128), dtype=torch.float32, device=DEV)
    sel = torch.empty((batch, c.groups, c.topk), dtype=torch.int32, device=DEV)
    cnt = torch.empty((batch, c.groups), dtype=torch.int32, device=DEV)
    Bd.kvs_decode_step_noalloc(c, pb.q, pb.k_pool, pb.v_pool, rp, pb.block_table, mb, pb.seq_lens, batch,
                               out, sel, cnt)
    return out, sel, cnt


def test_noalloc_matches_decode_step_twice():
    cases = [
        ("larger: 2 sequences, 2400-block rows, SEPARATE Quest k=64", 11, [2400 * B + 77, 1900 * B + 5],
         "separate", "quest", 64),
        ("smaller: 1 sequence of 60 blocks, SHARED Max k=16", 12, [60 * B + 17], "shared", "max", 16),
    ]
    for what, seed, lens, mode, rep, k in cases:
        say(f"[case] noalloc {what}")
        c, pb, rp = _case(seed, lens, mode, rep, k)
        need = kvs.kvs_decode_step_workspace_size(c, len(lens), pb.block_table.shape[1])
        assert need <= Bd.NOALLOC_SCRATCH_BYTES, need
        out_n, sel_n, cnt_n = _noalloc(c, pb, rp)
        out_w, sel_w, cnt_w = ops.decode_step(c, pb.q, pb.k_pool, pb.v_pool, rp, pb.block_table, pb.seq_lens)
        torch.cuda.synchronize()
        assert torch.equal(cnt_n, cnt_w), what
        for i in range(len(lens)):
            for gi in range(c.groups):
                n = int(cnt_w[i, gi])
                assert torch.equal(sel_n[i, gi, :n], sel_w[i, gi, :n]), (what, i, gi)
        err = float((out_n - out_w).abs().max())
        assert err <= ATOL, (what, err)
        say(f"[case] noalloc {what}: max |diff| {err:.2e}, bit-equal {torch.equal(out_n, out_w)}")


def test_noalloc_rejects_oversize_without_launch():
    c = kvs.Config(num_q_heads=32, num_kv_heads=8, initial_len=128, local_len=4096, topk=96,
                   rep_method="max", head_select_mode="separate")
    batch, mb = 64, 8192
    assert kvs.kvs_decode_step_workspace_size(c, batch, mb) > Bd.NOALLOC_SCRATCH_BYTES
    st = Bd.kvs_decode_step_noalloc(c, 0x10000, 0x10000, 0x10000, 0x10000, 0x10000, mb, 0x10000, batch,
                                    0x10000, None, None, stream=0, check=False)
    assert st == Bd.KVS_ERR_WORKSPACE
    assert "static scratch" in kvs.kvs_last_error()
