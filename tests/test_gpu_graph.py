"""Graph replays of the decode step against eager calls (needs an MI355X).

bench.py times kvs_decode_step (and kvs_decode_step_preselected) captured into a HIP graph and
replayed.  Here each captured step is replayed several times on different queries, with eager steps
on the same workspace in between, and every replay must equal the eager call on the same inputs bit
for bit: output, selection and count.  The step leaves its hand-off counters at zero, so a replay
needs no clearing node.  Shapes: the 128K headline layer (scoring, top-k and Initial/Local tiles in
one launch), a 2,400-block row (the wide top-k launch), Q4_0 and INT8 caches, and the confined
step.
"""
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

CASES = [
    # (name, L, rep, mode, k, kv, n_presel)
    ("128k-max", 131072, "max", "shared", 96, "fp16", 0),
    ("wide-quest", 2400 * 128 + 77, "quest", "separate", 64, "fp16", 0),
    ("128k-max-q4", 131072, "max", "shared", 96, "q4_0", 0),
    ("128k-presel", 131072, "max", "shared", 96, "fp16", 192),
    ("wide-quest-int8", 2400 * 128 + 77, "quest", "separate", 64, "int8_pth", 0),
    ("128k-max-int4", 131072, "max", "shared", 96, "int4_pth", 0),
]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("idx", range(len(CASES)), ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(idx):
    name, L, rep, mode, k, kv, n_presel = CASES[idx]
    say(f"[case] graph {name} L={L} rep={rep} mode={mode} k={k} kv={kv} presel={n_presel}")
    c = kvs.Config(num_q_heads=32, num_kv_heads=8, initial_len=128, local_len=4096, topk=k,
                   rep_method=rep, head_select_mode=mode, kv_type=kv)
    nb = (L + B - 1) // B
    seed = kvsynth.mix_seed(901, idx)
    q0, kp, vp, _ = kvsynth.pool_layer(seed, L, 32, 8, hot_range=(1, nb - 40), n_hot=20, device=DEV)
    ids = torch.arange(nb, dtype=torch.int32)
    if kv != "fp16":
        kp = ops.quantize_kv(c, kp, ids, ops.alloc_q8_pool(c, nb, DEV))
        vp = ops.quantize_kv(c, vp, ids, ops.alloc_q8_pool(c, nb, DEV))
    rp = ops.alloc_rep_pool(c, nb, DEV)
    ops.build_reps(c, kp, torch.arange(L // B, dtype=torch.int32), rp)
    table = torch.arange(nb, dtype=torch.int32, device=DEV).reshape(1, nb)
    lens = torch.tensor([L], dtype=torch.int32, device=DEV)
    qs = [q0[None].contiguous()] + [kvsynth.randn_fp16((1, 32, 128), kvsynth.mix_seed(seed, 50 + i), DEV)
                                    for i in range(3)]
    presel = None
    if n_presel:
        q_obs = kvsynth.randn_fp16((1, 32, 32, 128), kvsynth.mix_seed(seed, 60), DEV)
        imp = ops.token_importance(c, q_obs, kp, table, lens)
        presel, _ = ops.preselect_blocks(c, imp, lens, n_presel, nb)
        ws_bytes = kvs.kvs_decode_step_preselected_workspace_size(c, 1, nb, n_presel)
    else:
        ws_bytes = kvs.kvs_decode_step_workspace_size(c, 1, nb)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=DEV)  # hand-off counters start at zero
    out = torch.empty((1, 32, 128), dtype=torch.float32, device=DEV)
    sel = torch.empty((1, c.groups, k), dtype=torch.int32, device=DEV)
    cnt = torch.empty((1, c.groups), dtype=torch.int32, device=DEV)

    def step(q):  # on torch's current stream (the capture stream inside the graph block)
        if presel is not None:
            Bd.kvs_decode_step_preselected(c, q, kp, vp, rp, table, nb, lens, 1, presel, n_presel, out,
                                           sel, cnt, ws, ws_bytes)
        else:
            Bd.kvs_decode_step(c, q, kp, vp, rp, table, nb, lens, 1, out, sel, cnt, ws, ws_bytes)

    eager = []
    for q in qs:
        step(q)
        torch.cuda.synchronize()
        eager.append((out.clone(), sel.clone(), cnt.clone()))
    assert all(bool(torch.isfinite(e[0]).all()) for e in eager)

    q_static = torch.empty_like(qs[0])
    q_static.copy_(qs[0])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step(q_static)
    torch.cuda.synchronize()
    for rnd, i in enumerate([1, 0, 3, 2, 2]):
        step(qs[(i + 1) % len(qs)])  # an eager step on the same workspace between replays
        q_static.copy_(qs[i])
        out.fill_(float("nan"))
        sel.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o, sl, cn = eager[i]
        assert torch.equal(cnt, cn), f"{name} replay {rnd}: count {cnt.tolist()} vs {cn.tolist()}"
        assert torch.equal(sel, sl), f"{name} replay {rnd}: selection differs"
        assert torch.equal(out, o), f"{name} replay {rnd}: max |diff| {(out - o).abs().max().item()}"
    say(f"[ok] {name}: 5 replays equal the eager steps")
