"""The C ABI without a GPU: the library loads, exports every symbol include/kvs.h declares, and
rejects bad arguments on the host with the documented status before touching the device."""
import ctypes
import os
import re
import sys

import numpy as np

import pytest

import block_sparse_kv_amd as kvs
from block_sparse_kv_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvs.h")

ALIGNED = 0x10000        # fake device addresses: never dereferenced, every call below fails first
MISALIGNED = 0x10008


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvs_[a-z0-9_]+)\s*\(", src)))


def test_header_symbols_exported():
    lib = ctypes.CDLL(B.LIB_PATH)
    decl = declared_functions()
    assert len(decl) == 23, decl
    for name in decl:
        assert hasattr(lib, name), name
    assert sorted(B.EXPORTS) == decl


def test_config_struct_layout():
    assert ctypes.sizeof(B.kvs_config) == 48
    assert B.kvs_config.softmax_scale.offset == 40
    assert B.kvs_config.kv_type.offset == 44


def cfg(**kw):
    base = dict(num_q_heads=32, num_kv_heads=8, initial_len=128, local_len=4096, topk=96,
                rep_method="quest", head_select_mode="separate")
    base.update(kw)
    return kvs.Config(**base)


def test_status_strings():
    for st in (0, -1, -2, -3, -4, -5):
        assert kvs.kvs_status_string(st).startswith("KVS_")
    assert "unknown" in kvs.kvs_status_string(-99)


@pytest.mark.parametrize("kw,expect", [
    (dict(num_q_heads=0), B.KVS_ERR_INVALID_ARG),
    (dict(num_q_heads=30), B.KVS_ERR_INVALID_ARG),        # Hq % Hkv
    (dict(initial_len=-1), B.KVS_ERR_INVALID_ARG),
    (dict(local_len=-5), B.KVS_ERR_INVALID_ARG),
    (dict(topk=-1), B.KVS_ERR_INVALID_ARG),
    (dict(rep_method=7), B.KVS_ERR_INVALID_ARG),
    (dict(rep_method="dynamic", rep_num=0), B.KVS_ERR_INVALID_ARG),
    (dict(rep_method="dynamic", rep_num=129), B.KVS_ERR_INVALID_ARG),
    (dict(head_select_mode=3), B.KVS_ERR_INVALID_ARG),
    (dict(rep_method="fix", rep_num=3), B.KVS_ERR_INVALID_ARG),   # must divide 128
    (dict(rep_method="fix", rep_num=0), B.KVS_ERR_INVALID_ARG),
    (dict(softmax_scale=-1.0), B.KVS_ERR_INVALID_ARG),
    (dict(softmax_scale=float("nan")), B.KVS_ERR_INVALID_ARG),
    (dict(kv_type=5), B.KVS_ERR_INVALID_ARG),
    (dict(kv_type=-1), B.KVS_ERR_INVALID_ARG),
    (dict(head_dim=64), B.KVS_ERR_UNSUPPORTED),
    (dict(block_size=64), B.KVS_ERR_UNSUPPORTED),
    (dict(num_q_heads=48, num_kv_heads=3), B.KVS_ERR_UNSUPPORTED),
    (dict(num_q_heads=256, num_kv_heads=8), B.KVS_ERR_UNSUPPORTED),  # g = 32
])
def test_bad_config(kw, expect):
    c = cfg(**kw)
    assert kvs.kvs_rep_count(c) == expect
    assert kvs.kvs_rep_bytes_per_block(c) == 0
    assert kvs.kvs_kv_bytes_per_block(c) == 0
    assert kvs.kvs_attn_workspace_size(c, 1, 10) == 0
    assert kvs.kvs_decode_step_workspace_size(c, 1, 10) == 0
    A = ALIGNED
    assert kvs.kvs_build_reps(c, A, A, 4, A, stream=0, check=False) == expect
    assert kvs.kvs_quantize_kv(c, A, A, 4, A, stream=0, check=False) == expect
    assert kvs.kvs_score_blocks(c, A, A, A, 10, A, 1, A, stream=0, check=False) == expect
    assert kvs.kvs_topk_blocks(c, A, A, 1, 10, A, A, stream=0, check=False) == expect
    assert kvs.kvs_sparse_decode_attn(c, A, A, A, A, 10, A, 1, A, A, A, A, 1 << 30, stream=0,
                                      check=False) == expect
    assert kvs.kvs_decode_step(c, A, A, A, A, A, 10, A, 1, A, A, A, A, 1 << 30, stream=0,
                               check=False) == expect


def test_rep_counts_and_bytes():
    assert kvs.kvs_rep_count(cfg(rep_method="quest")) == 2
    assert kvs.kvs_rep_count(cfg(rep_method="max")) == 1
    assert kvs.kvs_rep_count(cfg(rep_method="mean")) == 1
    assert kvs.kvs_rep_count(cfg(rep_method="fix", rep_num=8)) == 8
    assert kvs.kvs_rep_bytes_per_block(cfg(rep_method="quest")) == 8 * 2 * 128 * 2
    assert kvs.kvs_rep_bytes_per_block(cfg(rep_method="mean")) == 8 * 1 * 128 * 4
    assert kvs.kvs_rep_bytes_per_block(cfg(rep_method="fix", rep_num=8)) == 8 * 8 * 128 * 2


def test_kv_bytes_and_quantize_errors():
    assert kvs.kvs_kv_bytes_per_block(cfg()) == 8 * 128 * 128 * 2
    q8 = cfg(kv_type="q8_0")
    assert kvs.kvs_kv_bytes_per_block(q8) == 8 * (128 * 128 + 128 * 4 * 2)
    assert kvs.kvs_kv_bytes_per_block(cfg(kv_type="q4_0")) == 8 * (128 * 64 + 128 * 4 * 2)
    assert kvs.kvs_kv_bytes_per_block(cfg(kv_type="int8_pth")) == 8 * (128 * 128 + 128 * 4)
    assert kvs.kvs_kv_bytes_per_block(cfg(kv_type="int4_pth")) == 8 * (128 * 64 + 128 * 4 + 128)
    A, M, Z = ALIGNED, MISALIGNED, None
    E = B.KVS_ERR_INVALID_ARG
    assert kvs.kvs_quantize_kv(cfg(), A, A, 3, A, stream=0, check=False) == E  # needs a quantized kv_type
    assert kvs.kvs_quantize_kv(q8, A, A, -1, A, stream=0, check=False) == E
    assert kvs.kvs_quantize_kv(q8, Z, A, 3, A, stream=0, check=False) == E
    assert kvs.kvs_quantize_kv(q8, A, A, 3, Z, stream=0, check=False) == E
    assert kvs.kvs_quantize_kv(q8, Z, Z, 0, Z, stream=0, check=False) == B.KVS_OK  # no-op
    assert kvs.kvs_quantize_kv(q8, M, A, 3, A, stream=0, check=False) == B.KVS_ERR_MISALIGNED
    assert kvs.kvs_quantize_kv(q8, A, A, 3, M, stream=0, check=False) == B.KVS_ERR_MISALIGNED
    assert kvs.kvs_quantize_kv(q8, A, A, 70000, A, stream=0, check=False) == B.KVS_ERR_UNSUPPORTED


def test_dynamic_rep_errors():
    dyn = cfg(rep_method="dynamic", rep_num=3)      # rep_num need not divide the block
    A, M, Z = ALIGNED, MISALIGNED, None
    E = B.KVS_ERR_INVALID_ARG
    assert kvs.kvs_rep_count(dyn) == 3
    assert kvs.kvs_rep_bytes_per_block(dyn) == 8 * 3 * 128 * 2
    assert kvs.kvs_build_reps(dyn, A, A, 3, A, stream=0, check=False) == E   # needs the scores
    assert kvs.kvs_build_dynamic_reps(cfg(), A, A, A, 10, A, 1, A, stream=0, check=False) == E
    assert kvs.kvs_build_dynamic_reps(dyn, A, Z, A, 10, A, 1, A, stream=0, check=False) == E
    assert kvs.kvs_build_dynamic_reps(dyn, M, A, A, 10, A, 1, A, stream=0, check=False) == B.KVS_ERR_MISALIGNED
    # a quantized cache passes the type check (the call still fails first, on the null scores)
    assert kvs.kvs_build_dynamic_reps(cfg(rep_method="dynamic", kv_type="q8_0"), A, Z, A, 10, A, 1, A,
                                      stream=0, check=False) == E
    need = kvs.kvs_importance_workspace_size(dyn, 2, 100, 16)
    assert need >= 2 * 8 * 16 * 4 * 100 * 8 and need % 256 == 0
    assert kvs.kvs_importance_workspace_size(dyn, 2, 100, 0) == 0
    assert kvs.kvs_importance_workspace_size(dyn, 2, 100, 4097) == 0
    run = lambda c, n, ws, wb, q=A: kvs.kvs_token_importance(c, q, n, A, A, 100, A, 2, A, ws, wb, stream=0,
                                                           check=False)
    assert run(dyn, 0, A, need) == E
    assert run(dyn, 5000, A, need) == B.KVS_ERR_UNSUPPORTED
    assert run(dyn, 16, A, need, q=Z) == E
    assert run(dyn, 16, A, need, q=M) == B.KVS_ERR_MISALIGNED
    assert run(dyn, 16, A, need - 256) == B.KVS_ERR_WORKSPACE
    assert run(dyn, 16, Z, need) == B.KVS_ERR_WORKSPACE
    assert run(dyn, 16, A + 16, need) == B.KVS_ERR_MISALIGNED
    assert run(cfg(kv_type="q8_0"), 16, A, need - 256) == B.KVS_ERR_WORKSPACE  # quantized: accepted


def test_preselect_errors():
    c = cfg()
    A, M, Z = ALIGNED, MISALIGNED, None
    E = B.KVS_ERR_INVALID_ARG
    need = kvs.kvs_preselect_workspace_size(c, 2, 100)
    assert need >= 2 * 8 * 100 * 4 and need % 256 == 0
    pre = lambda n, ws, wb, imp=A, pk=0: kvs.kvs_preselect_blocks(c, imp, A, 2, 100, n, pk, A, A, ws, wb,
                                                               stream=0, check=False)
    assert pre(0, A, need) == E
    assert pre(8, A, need, imp=Z) == E
    for pk in (-1, 2, 8, 128, 129):
        assert pre(8, A, need, pk=pk) == E
    assert pre(8, A, need, imp=A + 4, pk=5) == B.KVS_ERR_MISALIGNED
    assert pre(8, A, need - 256) == B.KVS_ERR_WORKSPACE
    assert pre(8, A + 16, need) == B.KVS_ERR_MISALIGNED
    need2 = kvs.kvs_decode_step_preselected_workspace_size(c, 2, 100, 32)
    assert need2 > kvs.kvs_attn_workspace_size(c, 2, 100)
    assert kvs.kvs_decode_step_preselected_workspace_size(c, 2, 100, 0) == 0
    step = lambda n, ws, wb, q=A, p=A: kvs.kvs_decode_step_preselected(
        c, q, A, A, A, A, 100, A, 2, p, n, A, None, None, ws, wb, stream=0, check=False)
    assert step(0, A, need2) == E
    assert step(32, A, need2, p=Z) == E
    assert step(32, A, need2, q=M) == B.KVS_ERR_MISALIGNED
    assert step(32, A, need2 - 256) == B.KVS_ERR_WORKSPACE
    assert step(32, Z, need2) == B.KVS_ERR_WORKSPACE


def test_null_and_size_errors():
    c = cfg()
    A, Z = ALIGNED, None
    E = B.KVS_ERR_INVALID_ARG
    assert kvs.kvs_build_reps(c, A, A, -1, A, stream=0, check=False) == E
    assert kvs.kvs_build_reps(c, Z, A, 3, A, stream=0, check=False) == E
    assert kvs.kvs_build_reps(c, Z, Z, 0, Z, stream=0, check=False) == B.KVS_OK  # no-op
    assert kvs.kvs_score_blocks(c, A, A, A, 0, A, 1, A, stream=0, check=False) == E
    assert kvs.kvs_score_blocks(c, A, A, A, 10, A, 0, A, stream=0, check=False) == E
    assert kvs.kvs_score_blocks(c, A, Z, A, 10, A, 1, A, stream=0, check=False) == E
    assert kvs.kvs_topk_blocks(c, A, A, 1, 10, Z, A, stream=0, check=False) == E
    assert kvs.kvs_sparse_decode_attn(c, A, A, Z, A, 10, A, 1, A, A, A, A, 1 << 30, stream=0,
                                      check=False) == E
    assert kvs.kvs_decode_step(c, A, A, A, A, A, 10, A, 1, Z, A, A, A, 1 << 30, stream=0,
                               check=False) == E


def test_alignment_and_workspace_errors():
    c = cfg()
    A, M = ALIGNED, MISALIGNED
    assert kvs.kvs_build_reps(c, M, A, 3, A, stream=0, check=False) == B.KVS_ERR_MISALIGNED
    assert kvs.kvs_score_blocks(c, M, A, A, 10, A, 1, A, stream=0, check=False) == \
        B.KVS_ERR_MISALIGNED
    need = kvs.kvs_attn_workspace_size(c, 2, 1024)
    assert need > 0 and need % 256 == 0
    assert kvs.kvs_sparse_decode_attn(c, A, A, A, A, 1024, A, 2, A, A, A, A, need - 1, stream=0,
                                      check=False) == B.KVS_ERR_WORKSPACE
    assert kvs.kvs_sparse_decode_attn(c, A, A, A, A, 1024, A, 2, A, A, A, None, need, stream=0,
                                      check=False) == B.KVS_ERR_WORKSPACE
    assert kvs.kvs_sparse_decode_attn(c, A, A, A, A, 1024, A, 2, A, A, A, A + 16, need, stream=0,
                                      check=False) == B.KVS_ERR_MISALIGNED
    need2 = kvs.kvs_decode_step_workspace_size(c, 2, 1024)
    assert need2 >= need + 2 * 8 * 1024 * 4
    assert kvs.kvs_decode_step(c, A, A, A, A, A, 1024, A, 2, A, None, None, A, need2 - 256,
                               stream=0, check=False) == B.KVS_ERR_WORKSPACE
    assert kvs.kvs_decode_step(c, A, A, A, M, A, 1024, A, 2, A, None, None, A, need2, stream=0,
                               check=False) == B.KVS_ERR_MISALIGNED


def test_decode_step_counter_limit():
    """The decode step keeps one hand-off counter per (sequence, group) in a fixed 64 KiB area:
    batch * G above 16384 is rejected before anything is enqueued."""
    c = cfg(head_select_mode="separate")  # G = 8
    A = ALIGNED
    assert kvs.kvs_decode_step(c, A, A, A, A, A, 64, A, 2049, A, None, None, A, 1 << 40, stream=0,
                               check=False) == B.KVS_ERR_UNSUPPORTED
    assert kvs.kvs_decode_step_workspace_size(c, 2048, 64) >= 65536


def test_workspace_grows_with_batch():
    c = cfg()
    a = kvs.kvs_decode_step_workspace_size(c, 1, 8192)
    b = kvs.kvs_decode_step_workspace_size(c, 16, 8192)
    assert 0 < a < b


def test_product_path_never_touches_oracle():
    """Nothing in the package imports or names the oracle; the library has no CPU fallback."""
    pkg = os.path.join(ROOT, "block_sparse_kv_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in src, f
                assert "kvsynth" not in src, f


def test_one_hip_runtime_in_process():
    """libkvs is bound to the HIP runtime torch loaded (one runtime per process)."""
    import torch  # noqa: F401
    maps = open("/proc/self/maps").read()
    hips = {ln.split()[-1] for ln in maps.splitlines() if "libamdhip64" in ln}
    assert len(hips) == 1, hips


# ------------------------------------------------------------------------------------------------
# Device-content rules (what KVS_DEBUG=1 checks), on host arrays: no GPU involved.
# ------------------------------------------------------------------------------------------------
def _contents_case():
    import numpy as np
    c = cfg(topk=4, initial_len=128, local_len=256, head_select_mode="shared")
    lens = np.array([20 * 128 + 5, 9 * 128], dtype=np.int32)      # candidates [1, 18) and [1, 7)
    table = np.arange(2 * 24, dtype=np.int32).reshape(2, 24)
    sel = np.array([[[3, 5, 17, -1]], [[1, 2, 6, -1]]], dtype=np.int32)
    cnt = np.array([[3], [3]], dtype=np.int32)
    presel = np.array([[[1, 4, -1]], [[2, 23, -1]]], dtype=np.int32)
    return c, lens, table, sel, cnt, presel


def test_contents_valid():
    c, lens, table, sel, cnt, presel = _contents_case()
    assert B.kvs_validate_contents(c, lens, 2, table, 24, sel, cnt, presel, 3) == B.KVS_OK
    assert B.kvs_validate_contents(c, lens, 2, None, 24) == B.KVS_OK


@pytest.mark.parametrize("what", ["len0", "len_over", "table_neg", "cnt_over_k", "cnt_over_cand", "cnt_neg",
                                  "sel_not_cand_low", "sel_in_local", "sel_repeat", "presel_low", "presel_high"])
def test_contents_rejected(what):
    c, lens, table, sel, cnt, presel = _contents_case()
    if what == "len0":
        lens[1] = 0
    elif what == "len_over":
        lens[0] = 24 * 128 + 1
    elif what == "table_neg":
        table[0, 20] = -1                     # block 20 holds the 5 last tokens of sequence 0
    elif what == "cnt_over_k":
        cnt[0, 0] = 5
    elif what == "cnt_over_cand":
        c = cfg(topk=8, initial_len=128, local_len=256, head_select_mode="shared")
        sel = np.concatenate([sel, np.full((2, 1, 4), -1, np.int32)], axis=2)
        sel[1, 0, :7] = [1, 2, 3, 4, 5, 6, 6]
        cnt[1, 0] = 7                         # sequence 1 has 6 candidates
    elif what == "cnt_neg":
        cnt[1, 0] = -1
    elif what == "sel_not_cand_low":
        sel[0, 0, 0] = 0                      # the Initial block
    elif what == "sel_in_local":
        sel[1, 0, 2] = 7                      # sequence 1's Local starts at block 7
    elif what == "sel_repeat":
        sel[0, 0, 1] = 3
    elif what == "presel_low":
        presel[0, 0, 2] = -2
    elif what == "presel_high":
        presel[1, 0, 0] = 24
    st = B.kvs_validate_contents(c, np.ascontiguousarray(lens), 2, np.ascontiguousarray(table), 24,
                                 np.ascontiguousarray(sel), np.ascontiguousarray(cnt),
                                 np.ascontiguousarray(presel), 3)
    assert st == B.KVS_ERR_INVALID_ARG, what
    assert "kvs contents" in kvs.kvs_last_error()


def test_contents_bad_arguments():
    c, lens, table, sel, cnt, presel = _contents_case()
    assert B.kvs_validate_contents(c, None, 2, table, 24) == B.KVS_ERR_INVALID_ARG
    assert B.kvs_validate_contents(c, lens, 0, table, 24) == B.KVS_ERR_INVALID_ARG
    assert B.kvs_validate_contents(c, lens, 2, table, 24, sel, None) == B.KVS_ERR_INVALID_ARG


def test_noalloc_host_checks():
    """kvs_decode_step_noalloc rejects bad arguments and sizes beyond its static scratch on the host,
    before any HIP call."""
    c = cfg(topk=96, rep_method="max")
    st = B.kvs_decode_step_noalloc(c, None, ALIGNED, ALIGNED, ALIGNED, ALIGNED, 1024, ALIGNED, 1,
                                   ALIGNED, None, None, stream=0, check=False)
    assert st == B.KVS_ERR_INVALID_ARG
    st = B.kvs_decode_step_noalloc(c, MISALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, 1024, ALIGNED, 1,
                                   ALIGNED, None, None, stream=0, check=False)
    assert st == B.KVS_ERR_MISALIGNED
    assert kvs.kvs_decode_step_workspace_size(c, 64, 8192) > B.NOALLOC_SCRATCH_BYTES
    st = B.kvs_decode_step_noalloc(c, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, 8192, ALIGNED, 64,
                                   ALIGNED, None, None, stream=0, check=False)
    assert st == B.KVS_ERR_WORKSPACE
    assert "static scratch" in kvs.kvs_last_error()


def test_gather_read_floor_host_checks():
    """kvs_gather_read_floor rejects bad sizes and pointers on the host; no tiles enqueue nothing."""
    f = B.kvs_gather_read_floor
    assert f(ALIGNED, ALIGNED, 8, ALIGNED, -1, 0, ALIGNED, stream=0, check=False) == B.KVS_ERR_INVALID_ARG
    assert f(ALIGNED, ALIGNED, -1, ALIGNED, 4, 0, ALIGNED, stream=0, check=False) == B.KVS_ERR_INVALID_ARG
    assert f(ALIGNED, ALIGNED, 8, ALIGNED, 4, -1, ALIGNED, stream=0, check=False) == B.KVS_ERR_INVALID_ARG
    assert f(ALIGNED, ALIGNED, 8, ALIGNED, 4, 65537, ALIGNED, stream=0, check=False) == B.KVS_ERR_INVALID_ARG
    assert f(ALIGNED, ALIGNED, 8, None, 4, 0, ALIGNED, stream=0, check=False) == B.KVS_ERR_INVALID_ARG
    assert f(ALIGNED, None, 8, ALIGNED, 4, 0, ALIGNED, stream=0, check=False) == B.KVS_ERR_INVALID_ARG
    assert f(MISALIGNED, ALIGNED, 8, ALIGNED, 4, 0, ALIGNED, stream=0, check=False) == B.KVS_ERR_MISALIGNED
    assert f(None, None, 0, None, 0, 0, None, stream=0, check=False) == B.KVS_OK


def test_timeline_variant_exports():
    """The timeline library (build.py --timeline) exports every entry point plus kvs_timeline_set; the
    default library carries no timeline code."""
    import ctypes
    import subprocess

    here = os.path.dirname(B.LIB_PATH)
    assert not hasattr(ctypes.CDLL(os.path.join(here, "libkvs.so")), "kvs_timeline_set")
    tl = os.path.join(here, "libkvs_timeline.so")
    if not os.path.exists(tl):
        pytest.skip("libkvs_timeline.so not built")
    code = ("import block_sparse_kv_amd.binding as b; assert b.TIMELINE and b.LIB_PATH.endswith("
            "'libkvs_timeline.so'); [getattr(b._lib, n) for n in b.EXPORTS]; b._lib.kvs_timeline_set; "
            "print('ok')")
    env = dict(os.environ, KVS_LIBRARY="timeline")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       cwd=os.path.dirname(here))
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stderr[-2000:]
    env["KVS_LIBRARY"] = "bogus"
    r = subprocess.run([sys.executable, "-c", "import block_sparse_kv_amd"], env=env, capture_output=True,
                       text=True, cwd=os.path.dirname(here))
    assert r.returncode != 0 and "KVS_LIBRARY" in r.stderr
