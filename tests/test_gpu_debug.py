"""KVS_DEBUG=1 (needs an MI355X): with valid device contents, every entry point that checks them
gives results bit-identical to the same call without the check.  Contents that break the rules are
exercised on the CPU only (tests/test_abi_cpu.py, kvs_validate_contents on host arrays): no kernel is
ever launched here with bad contents."""
from __future__ import annotations

import os
import sys

import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("no GPU", allow_module_level=True)

import block_sparse_kv_amd as kvs  # noqa: E402
from block_sparse_kv_amd import ops  # noqa: E402

import kvsynth  # noqa: E402

DEV = "cuda"
B = 128


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture
def debug_env():
    old = os.environ.get("KVS_DEBUG")
    yield
    if old is None:
        os.environ.pop("KVS_DEBUG", None)
    else:
        os.environ["KVS_DEBUG"] = old


@pytest.mark.parametrize("L,mode", [(40 * 128 + 17, "separate"), (3000 * 128 + 5, "shared")])
def test_debug_mode_bit_identical(debug_env, L, mode):
    say(f"[case] KVS_DEBUG bit identity L={L} mode={mode}")
    c = kvs.Config(num_q_heads=32, num_kv_heads=8, initial_len=128, local_len=1024, topk=16,
                   rep_method="quest", head_select_mode=mode)
    s1 = kvsynth.make_sequence(kvsynth.mix_seed(77, L), L, 32, 8, device=DEV)
    s2 = kvsynth.make_sequence(kvsynth.mix_seed(78, L), L - 300, 32, 8, device=DEV)
    pb = kvsynth.page_batch([s1, s2], B, shuffle_seed=5, spare_blocks=3, device=DEV)
    n_phys = pb.k_pool.shape[0]
    ids = torch.cat([pb.block_table[i, : int(pb.seq_lens[i]) // B] for i in range(2)]).cpu()
    results = {}
    for dbg in ("0", "1"):
        os.environ["KVS_DEBUG"] = dbg
        rp = ops.alloc_rep_pool(c, n_phys, DEV)
        ops.build_reps(c, pb.k_pool, ids, rp)
        sc = ops.score_blocks(c, pb.q, rp, pb.block_table, pb.seq_lens)
        sel, cnt = ops.topk_blocks(c, sc, pb.seq_lens)
        att = ops.sparse_decode_attn(c, pb.q, pb.k_pool, pb.v_pool, pb.block_table, pb.seq_lens, sel, cnt)
        out, sel2, cnt2 = ops.decode_step(c, pb.q, pb.k_pool, pb.v_pool, rp, pb.block_table, pb.seq_lens)
        torch.cuda.synchronize()
        built = rp.index_select(0, ids.to(DEV).long())  # blocks never built hold whatever was there
        results[dbg] = [t.clone() for t in (built, sc, sel, cnt, att, out, sel2, cnt2)]
    names = ("reps", "scores", "sel", "cnt", "attn", "step out", "step sel", "step cnt")
    for n, a, b in zip(names, results["0"], results["1"]):
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.float16 else a,
                           b.view(torch.uint8) if b.dtype == torch.float16 else b), n
    say(f"[case] KVS_DEBUG bit identity L={L} mode={mode}: ok")
