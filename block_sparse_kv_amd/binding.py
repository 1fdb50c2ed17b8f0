"""ctypes binding of libkvs.so: the C entry points under the same names, argument marshalling only.

Tensors are passed as their data pointers, the stream as torch's current HIP stream (or an explicit
``stream`` handle).  Every computation happens in the library's HIP kernels; nothing here computes.
A missing library is an ImportError: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
# KVS_LIBRARY=timeline loads the variant with per-workgroup timeline records (build.py --timeline)
_VARIANTS = {"": ("libkvs.so", ""), "timeline": ("libkvs_timeline.so", " --timeline")}
_variant = os.environ.get("KVS_LIBRARY", "")
if _variant not in _VARIANTS:
    raise ImportError(f"KVS_LIBRARY={_variant!r}: expected unset or 'timeline'")
LIB_PATH = os.path.join(HERE, _VARIANTS[_variant][0])
TIMELINE = _variant == "timeline"

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run `python block_sparse_kv_amd/build.py"
                      f"{_VARIANTS[_variant][1]}` (or __graft_entry__.build()) first")
# torch must be loaded first: its bundled HIP runtime has the SONAME libamdhip64.so.7 that libkvs
# needs, so the loader binds libkvs to that same runtime.  Loading libkvs first would bring in a
# second HIP runtime, and torch's streams and device memory would mean nothing to it.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

KVS_OK, KVS_ERR_INVALID_ARG, KVS_ERR_UNSUPPORTED, KVS_ERR_MISALIGNED, KVS_ERR_WORKSPACE, \
    KVS_ERR_HIP = 0, -1, -2, -3, -4, -5
REP_QUEST, REP_MAX, REP_MEAN, REP_FIX, REP_DYNAMIC = 0, 1, 2, 3, 4
HEADS_SEPARATE, HEADS_SHARED = 0, 1
KV_FP16, KV_Q8_0, KV_Q4_0, KV_INT8_PTH, KV_INT4_PTH = 0, 1, 2, 3, 4
KV_NAMES = {"fp16": KV_FP16, "q8_0": KV_Q8_0, "q4_0": KV_Q4_0, "int8_pth": KV_INT8_PTH,
            "int4_pth": KV_INT4_PTH}
REP_NAMES = {"quest": REP_QUEST, "max": REP_MAX, "mean": REP_MEAN, "fix": REP_FIX,
             "dynamic": REP_DYNAMIC}
MODE_NAMES = {"separate": HEADS_SEPARATE, "shared": HEADS_SHARED}

EXPORTS = (
    "kvs_status_string", "kvs_last_error", "kvs_rep_count", "kvs_rep_bytes_per_block",
    "kvs_kv_bytes_per_block", "kvs_quantize_kv", "kvs_build_reps", "kvs_importance_workspace_size",
    "kvs_token_importance", "kvs_build_dynamic_reps", "kvs_preselect_workspace_size",
    "kvs_preselect_blocks", "kvs_decode_step_preselected_workspace_size", "kvs_decode_step_preselected",
    "kvs_score_blocks", "kvs_topk_blocks", "kvs_attn_workspace_size", "kvs_sparse_decode_attn",
    "kvs_decode_step_workspace_size", "kvs_decode_step", "kvs_validate_contents",
    "kvs_decode_step_noalloc", "kvs_gather_read_floor",
)
NOALLOC_SCRATCH_BYTES = 32 << 20  # KVS_NOALLOC_SCRATCH_BYTES


class kvs_config(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("initial_len", ctypes.c_int32), ("local_len", ctypes.c_int32),
        ("topk", ctypes.c_int32), ("rep_method", ctypes.c_int32), ("rep_num", ctypes.c_int32),
        ("head_select_mode", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("kv_type", ctypes.c_int32),
    ]


@dataclass
class Config:
    """Python mirror of kvs_config; rep_method / head_select_mode / kv_type accept names or codes."""
    num_q_heads: int
    num_kv_heads: int
    initial_len: int
    local_len: int
    topk: int
    rep_method: object = "quest"
    rep_num: int = 1
    head_select_mode: object = "separate"
    head_dim: int = 128
    block_size: int = 128
    softmax_scale: float = 0.0
    kv_type: object = "fp16"

    def c(self) -> kvs_config:
        rm = REP_NAMES.get(self.rep_method, self.rep_method)
        hm = MODE_NAMES.get(self.head_select_mode, self.head_select_mode)
        kt = KV_NAMES.get(self.kv_type, self.kv_type)
        return kvs_config(self.num_q_heads, self.num_kv_heads, self.head_dim, self.block_size,
                          self.initial_len, self.local_len, self.topk, int(rm), self.rep_num,
                          int(hm), float(self.softmax_scale), int(kt))

    @property
    def groups(self) -> int:
        hm = MODE_NAMES.get(self.head_select_mode, self.head_select_mode)
        return self.num_kv_heads if hm == HEADS_SEPARATE else 1


_P = ctypes.c_void_p
_I = ctypes.c_int32
_S = ctypes.c_size_t
_CFG = ctypes.POINTER(kvs_config)
_lib.kvs_status_string.restype = ctypes.c_char_p
_lib.kvs_status_string.argtypes = [ctypes.c_int]
_lib.kvs_last_error.restype = ctypes.c_char_p
_lib.kvs_last_error.argtypes = []
_lib.kvs_rep_count.restype = ctypes.c_int
_lib.kvs_rep_count.argtypes = [_CFG]
_lib.kvs_rep_bytes_per_block.restype = _S
_lib.kvs_rep_bytes_per_block.argtypes = [_CFG]
_lib.kvs_kv_bytes_per_block.restype = _S
_lib.kvs_kv_bytes_per_block.argtypes = [_CFG]
_lib.kvs_quantize_kv.restype = ctypes.c_int
_lib.kvs_quantize_kv.argtypes = [_CFG, _P, _P, _I, _P, _P]
_lib.kvs_build_reps.restype = ctypes.c_int
_lib.kvs_build_reps.argtypes = [_CFG, _P, _P, _I, _P, _P]
_lib.kvs_importance_workspace_size.restype = _S
_lib.kvs_importance_workspace_size.argtypes = [_CFG, _I, _I, _I]
_lib.kvs_token_importance.restype = ctypes.c_int
_lib.kvs_token_importance.argtypes = [_CFG, _P, _I, _P, _P, _I, _P, _I, _P, _P, _S, _P]
_lib.kvs_build_dynamic_reps.restype = ctypes.c_int
_lib.kvs_build_dynamic_reps.argtypes = [_CFG, _P, _P, _P, _I, _P, _I, _P, _P]
_lib.kvs_preselect_workspace_size.restype = _S
_lib.kvs_preselect_workspace_size.argtypes = [_CFG, _I, _I]
_lib.kvs_preselect_blocks.restype = ctypes.c_int
_lib.kvs_preselect_blocks.argtypes = [_CFG, _P, _P, _I, _I, _I, _I, _P, _P, _P, _S, _P]
_lib.kvs_decode_step_preselected_workspace_size.restype = _S
_lib.kvs_decode_step_preselected_workspace_size.argtypes = [_CFG, _I, _I, _I]
_lib.kvs_decode_step_preselected.restype = ctypes.c_int
_lib.kvs_decode_step_preselected.argtypes = [_CFG, _P, _P, _P, _P, _P, _I, _P, _I, _P, _I, _P, _P, _P, _P, _S, _P]
_lib.kvs_score_blocks.restype = ctypes.c_int
_lib.kvs_score_blocks.argtypes = [_CFG, _P, _P, _P, _I, _P, _I, _P, _P]
_lib.kvs_topk_blocks.restype = ctypes.c_int
_lib.kvs_topk_blocks.argtypes = [_CFG, _P, _P, _I, _I, _P, _P, _P]
_lib.kvs_attn_workspace_size.restype = _S
_lib.kvs_attn_workspace_size.argtypes = [_CFG, _I, _I]
_lib.kvs_sparse_decode_attn.restype = ctypes.c_int
_lib.kvs_sparse_decode_attn.argtypes = [_CFG, _P, _P, _P, _P, _I, _P, _I, _P, _P, _P, _P, _S, _P]
_lib.kvs_decode_step_workspace_size.restype = _S
_lib.kvs_decode_step_workspace_size.argtypes = [_CFG, _I, _I]
_lib.kvs_decode_step.restype = ctypes.c_int
_lib.kvs_decode_step.argtypes = [_CFG, _P, _P, _P, _P, _P, _I, _P, _I, _P, _P, _P, _P, _S, _P]
_lib.kvs_decode_step_noalloc.restype = ctypes.c_int
_lib.kvs_decode_step_noalloc.argtypes = [_CFG, _P, _P, _P, _P, _P, _I, _P, _I, _P, _P, _P, _P]
_lib.kvs_gather_read_floor.restype = ctypes.c_int
_lib.kvs_gather_read_floor.argtypes = [_P, _P, _I, _P, _I, _I, _P, _P]
_lib.kvs_validate_contents.restype = ctypes.c_int
_lib.kvs_validate_contents.argtypes = [_CFG, _P, _I, _P, _I, _P, _P, _P, _I]


class KvsError(RuntimeError):
    def __init__(self, status: int, where: str):
        detail = kvs_last_error() if status == KVS_ERR_HIP else ""
        super().__init__(f"{where}: {kvs_status_string(status)} ({status}) {detail}".rstrip())
        self.status = status


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _cfg(cfg):
    return ctypes.byref(cfg.c() if isinstance(cfg, Config) else cfg)


def _check(st: int, where: str) -> int:
    if st != KVS_OK:
        raise KvsError(st, where)
    return st


def kvs_status_string(status: int) -> str:
    return _lib.kvs_status_string(status).decode()


def kvs_last_error() -> str:
    return _lib.kvs_last_error().decode()


def kvs_rep_count(cfg) -> int:
    return _lib.kvs_rep_count(_cfg(cfg))


def kvs_rep_bytes_per_block(cfg) -> int:
    return _lib.kvs_rep_bytes_per_block(_cfg(cfg))


def kvs_kv_bytes_per_block(cfg) -> int:
    return _lib.kvs_kv_bytes_per_block(_cfg(cfg))


def kvs_quantize_kv(cfg, src_pool, phys_block_ids, n_blocks, dst_pool, stream=None, check=True):
    st = _lib.kvs_quantize_kv(_cfg(cfg), _ptr(src_pool), _ptr(phys_block_ids), n_blocks,
                              _ptr(dst_pool), _stream(stream))
    return _check(st, "kvs_quantize_kv") if check else st


def kvs_build_reps(cfg, k_pool, phys_block_ids, n_blocks, rep_pool, stream=None, check=True):
    st = _lib.kvs_build_reps(_cfg(cfg), _ptr(k_pool), _ptr(phys_block_ids), n_blocks,
                             _ptr(rep_pool), _stream(stream))
    return _check(st, "kvs_build_reps") if check else st


def kvs_importance_workspace_size(cfg, batch, max_blocks_per_seq, n_obs) -> int:
    return _lib.kvs_importance_workspace_size(_cfg(cfg), batch, max_blocks_per_seq, n_obs)


def kvs_token_importance(cfg, q_obs, n_obs, k_pool, block_table, max_blocks_per_seq, seq_lens, batch,
                         importance, workspace, workspace_bytes, stream=None, check=True):
    st = _lib.kvs_token_importance(_cfg(cfg), _ptr(q_obs), n_obs, _ptr(k_pool), _ptr(block_table),
                                   max_blocks_per_seq, _ptr(seq_lens), batch, _ptr(importance),
                                   _ptr(workspace), workspace_bytes, _stream(stream))
    return _check(st, "kvs_token_importance") if check else st


def kvs_build_dynamic_reps(cfg, k_pool, importance, block_table, max_blocks_per_seq, seq_lens, batch,
                           rep_pool, stream=None, check=True):
    st = _lib.kvs_build_dynamic_reps(_cfg(cfg), _ptr(k_pool), _ptr(importance), _ptr(block_table),
                                     max_blocks_per_seq, _ptr(seq_lens), batch, _ptr(rep_pool),
                                     _stream(stream))
    return _check(st, "kvs_build_dynamic_reps") if check else st


def kvs_preselect_workspace_size(cfg, batch, max_blocks_per_seq) -> int:
    return _lib.kvs_preselect_workspace_size(_cfg(cfg), batch, max_blocks_per_seq)


def kvs_preselect_blocks(cfg, importance, seq_lens, batch, max_blocks_per_seq, n_presel, pool_kernel,
                         presel, presel_count, workspace, workspace_bytes, stream=None, check=True):
    st = _lib.kvs_preselect_blocks(_cfg(cfg), _ptr(importance), _ptr(seq_lens), batch,
                                   max_blocks_per_seq, n_presel, pool_kernel, _ptr(presel),
                                   _ptr(presel_count),
                                   _ptr(workspace), workspace_bytes, _stream(stream))
    return _check(st, "kvs_preselect_blocks") if check else st


def kvs_decode_step_preselected_workspace_size(cfg, batch, max_blocks_per_seq, n_presel) -> int:
    return _lib.kvs_decode_step_preselected_workspace_size(_cfg(cfg), batch, max_blocks_per_seq, n_presel)


def kvs_decode_step_preselected(cfg, q, k_pool, v_pool, rep_pool, block_table, max_blocks_per_seq,
                                seq_lens, batch, presel, n_presel, out, sel_out, sel_count_out,
                                workspace, workspace_bytes, stream=None, check=True):
    st = _lib.kvs_decode_step_preselected(_cfg(cfg), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                          _ptr(rep_pool), _ptr(block_table), max_blocks_per_seq,
                                          _ptr(seq_lens), batch, _ptr(presel), n_presel, _ptr(out),
                                          _ptr(sel_out), _ptr(sel_count_out), _ptr(workspace),
                                          workspace_bytes, _stream(stream))
    return _check(st, "kvs_decode_step_preselected") if check else st


def kvs_score_blocks(cfg, q, rep_pool, block_table, max_blocks_per_seq, seq_lens, batch, scores,
                     stream=None, check=True):
    st = _lib.kvs_score_blocks(_cfg(cfg), _ptr(q), _ptr(rep_pool), _ptr(block_table),
                               max_blocks_per_seq, _ptr(seq_lens), batch, _ptr(scores),
                               _stream(stream))
    return _check(st, "kvs_score_blocks") if check else st


def kvs_topk_blocks(cfg, scores, seq_lens, batch, max_blocks_per_seq, sel, sel_count,
                    stream=None, check=True):
    st = _lib.kvs_topk_blocks(_cfg(cfg), _ptr(scores), _ptr(seq_lens), batch,
                              max_blocks_per_seq, _ptr(sel), _ptr(sel_count), _stream(stream))
    return _check(st, "kvs_topk_blocks") if check else st


def kvs_attn_workspace_size(cfg, batch, max_blocks_per_seq) -> int:
    return _lib.kvs_attn_workspace_size(_cfg(cfg), batch, max_blocks_per_seq)


def kvs_sparse_decode_attn(cfg, q, k_pool, v_pool, block_table, max_blocks_per_seq, seq_lens,
                           batch, sel, sel_count, out, workspace, workspace_bytes, stream=None,
                           check=True):
    st = _lib.kvs_sparse_decode_attn(_cfg(cfg), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                     _ptr(block_table), max_blocks_per_seq, _ptr(seq_lens), batch,
                                     _ptr(sel), _ptr(sel_count), _ptr(out), _ptr(workspace),
                                     workspace_bytes, _stream(stream))
    return _check(st, "kvs_sparse_decode_attn") if check else st


def kvs_decode_step_workspace_size(cfg, batch, max_blocks_per_seq) -> int:
    return _lib.kvs_decode_step_workspace_size(_cfg(cfg), batch, max_blocks_per_seq)


def kvs_decode_step(cfg, q, k_pool, v_pool, rep_pool, block_table, max_blocks_per_seq, seq_lens,
                    batch, out, sel_out, sel_count_out, workspace, workspace_bytes, stream=None,
                    check=True):
    st = _lib.kvs_decode_step(_cfg(cfg), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(rep_pool),
                              _ptr(block_table), max_blocks_per_seq, _ptr(seq_lens), batch,
                              _ptr(out), _ptr(sel_out), _ptr(sel_count_out), _ptr(workspace),
                              workspace_bytes, _stream(stream))
    return _check(st, "kvs_decode_step") if check else st


def kvs_validate_contents(cfg, seq_lens, batch, block_table, max_blocks_per_seq, sel=None, sel_count=None,
                          presel=None, n_presel=0) -> int:
    """Host arrays (numpy int32, C-contiguous) or raw host addresses; returns the status (no raise)."""
    def hp(a):
        if a is None or isinstance(a, int):
            return a
        assert a.dtype.name == "int32" and a.flags["C_CONTIGUOUS"], "int32 C-contiguous host array"
        return a.ctypes.data
    return _lib.kvs_validate_contents(_cfg(cfg), hp(seq_lens), batch, hp(block_table), max_blocks_per_seq,
                                      hp(sel), hp(sel_count), hp(presel), n_presel)


def kvs_decode_step_noalloc(cfg, q, k_pool, v_pool, rep_pool, block_table, max_blocks_per_seq, seq_lens,
                            batch, out, sel_out, sel_count_out, stream=None, check=True):
    st = _lib.kvs_decode_step_noalloc(_cfg(cfg), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(rep_pool),
                                      _ptr(block_table), max_blocks_per_seq, _ptr(seq_lens), batch,
                                      _ptr(out), _ptr(sel_out), _ptr(sel_count_out), _stream(stream))
    return _check(st, "kvs_decode_step_noalloc") if check else st


def kvs_gather_read_floor(k_pool, v_pool, pool_tiles, tile_ids, n_tiles, lds_bytes, out, stream=None,
                          check=True):
    st = _lib.kvs_gather_read_floor(_ptr(k_pool), _ptr(v_pool), pool_tiles, _ptr(tile_ids), n_tiles,
                                    lds_bytes, _ptr(out), _stream(stream))
    return _check(st, "kvs_gather_read_floor") if check else st


if TIMELINE:
    _lib.kvs_timeline_set.restype = None
    _lib.kvs_timeline_set.argtypes = [_P]


def kvs_timeline_set(records):
    """Timeline library only: the device record array later calls write into (None stops)."""
    if not TIMELINE:
        raise RuntimeError("kvs_timeline_set needs the timeline library (KVS_LIBRARY=timeline)")
    _lib.kvs_timeline_set(_ptr(records))

