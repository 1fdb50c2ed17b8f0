"""Torch-facing helpers over the C entry points: allocate outputs and workspaces as torch tensors on
the inputs' device and call libkvs on torch's current stream.  No arithmetic happens here."""
from __future__ import annotations

import torch

from . import binding as B


def _rep_dtype(cfg: B.Config):
    return torch.float32 if B.REP_NAMES.get(cfg.rep_method, cfg.rep_method) == B.REP_MEAN \
        else torch.float16


def alloc_rep_pool(cfg: B.Config, n_phys: int, device) -> torch.Tensor:
    """[n_phys][Hkv][R][128] in fp16 (fp32 for Mean)."""
    R = B.kvs_rep_count(cfg)
    if R < 0:
        raise B.KvsError(R, "alloc_rep_pool")
    return torch.empty((n_phys, cfg.num_kv_heads, R, cfg.head_dim), dtype=_rep_dtype(cfg),
                       device=device)


def alloc_q8_pool(cfg: B.Config, n_phys: int, device) -> torch.Tensor:
    """A quantized K or V pool of cfg.kv_type as bytes [n_phys][Hkv][record]: Q8_0 records of 17408
    bytes (int8 codes [128][128] + fp16 scales [128][4]), Q4_0 records of 9216 bytes."""
    per_block = B.kvs_kv_bytes_per_block(cfg)
    if per_block == 0:
        raise B.KvsError(B.KVS_ERR_INVALID_ARG, "alloc_q8_pool")
    return torch.empty((n_phys, cfg.num_kv_heads, per_block // cfg.num_kv_heads), dtype=torch.uint8,
                       device=device)


def quantize_kv(cfg, src_pool, phys_ids: torch.Tensor, dst_pool: torch.Tensor):
    ids = phys_ids.to(device=src_pool.device, dtype=torch.int32).contiguous()
    B.kvs_quantize_kv(cfg, src_pool, ids, ids.numel(), dst_pool)
    return dst_pool


def build_reps(cfg, k_pool, phys_ids: torch.Tensor, rep_pool: torch.Tensor):
    ids = phys_ids.to(device=k_pool.device, dtype=torch.int32).contiguous()
    B.kvs_build_reps(cfg, k_pool, ids, ids.numel(), rep_pool)
    return rep_pool


def token_importance(cfg, q_obs, k_pool, block_table, seq_lens):
    """q_obs [batch][n_obs][Hq][128] fp16 -> importance [batch][G][max_blocks * 128] fp32."""
    batch, mb = block_table.shape
    n_obs = q_obs.shape[1]
    imp = torch.empty((batch, cfg.groups, mb * 128), dtype=torch.float32, device=q_obs.device)
    need = B.kvs_importance_workspace_size(cfg, batch, mb, n_obs)
    ws = workspace(need, q_obs.device)
    B.kvs_token_importance(cfg, q_obs.contiguous(), n_obs, k_pool, block_table, mb, seq_lens, batch,
                           imp, ws, ws.numel())
    return imp


def build_dynamic_reps(cfg, k_pool, importance, block_table, seq_lens, rep_pool):
    batch, mb = block_table.shape
    B.kvs_build_dynamic_reps(cfg, k_pool, importance, block_table, mb, seq_lens, batch, rep_pool)
    return rep_pool


def preselect_blocks(cfg, importance, seq_lens, n_presel, max_blocks, pool_kernel=0):
    batch = seq_lens.shape[0]
    presel = torch.empty((batch, cfg.groups, n_presel), dtype=torch.int32, device=importance.device)
    cnt = torch.empty((batch, cfg.groups), dtype=torch.int32, device=importance.device)
    ws = workspace(B.kvs_preselect_workspace_size(cfg, batch, max_blocks), importance.device)
    B.kvs_preselect_blocks(cfg, importance, seq_lens, batch, max_blocks, n_presel, pool_kernel, presel,
                           cnt, ws, ws.numel())
    return presel, cnt


def decode_step_preselected(cfg, q, k_pool, v_pool, rep_pool, block_table, seq_lens, presel):
    batch, mb = block_table.shape
    n_presel = presel.shape[-1]
    out = torch.empty((batch, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32, device=q.device)
    sel = torch.empty((batch, cfg.groups, max(cfg.topk, 1)), dtype=torch.int32, device=q.device)
    cnt = torch.empty((batch, cfg.groups), dtype=torch.int32, device=q.device)
    # zeroed: its first bytes are the hand-off counters, which every completed call leaves zero
    ws = torch.zeros(B.kvs_decode_step_preselected_workspace_size(cfg, batch, mb, n_presel), dtype=torch.uint8,
                     device=q.device)
    B.kvs_decode_step_preselected(cfg, q, k_pool, v_pool, rep_pool, block_table, mb, seq_lens, batch,
                                  presel.contiguous(), n_presel, out, sel, cnt, ws, ws.numel())
    return out, sel[:, :, : cfg.topk], cnt


def score_blocks(cfg, q, rep_pool, block_table, seq_lens):
    batch, mb = block_table.shape
    scores = torch.empty((batch, cfg.groups, mb), dtype=torch.float32, device=q.device)
    B.kvs_score_blocks(cfg, q, rep_pool, block_table, mb, seq_lens, batch, scores)
    return scores


def topk_blocks(cfg, scores, seq_lens):
    batch, G, mb = scores.shape
    sel = torch.empty((batch, G, max(cfg.topk, 1)), dtype=torch.int32, device=scores.device)
    cnt = torch.empty((batch, G), dtype=torch.int32, device=scores.device)
    B.kvs_topk_blocks(cfg, scores, seq_lens, batch, mb, sel, cnt)
    return sel[:, :, : cfg.topk], cnt


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def sparse_decode_attn(cfg, q, k_pool, v_pool, block_table, seq_lens, sel, sel_count, ws=None):
    batch, mb = block_table.shape
    out = torch.empty((batch, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32, device=q.device)
    need = B.kvs_attn_workspace_size(cfg, batch, mb)
    if ws is None:
        ws = workspace(need, q.device)
    B.kvs_sparse_decode_attn(cfg, q, k_pool, v_pool, block_table, mb, seq_lens, batch,
                             sel.contiguous() if cfg.topk > 0 else None, sel_count, out, ws,
                             ws.numel())
    return out


def step_workspace(cfg, batch, max_blocks, device) -> torch.Tensor:
    """A zero-filled kvs_decode_step workspace (its hand-off counters must start at zero).  Use it
    for kvs_decode_step only, and zero it again after a call that failed or did not complete."""
    n = max(B.kvs_decode_step_workspace_size(cfg, batch, max_blocks), 256)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def decode_step(cfg, q, k_pool, v_pool, rep_pool, block_table, seq_lens, ws=None):
    """ws, if given, must hold kvs_decode_step_workspace_size bytes (step_workspace)."""
    batch, mb = block_table.shape
    out = torch.empty((batch, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32, device=q.device)
    sel = torch.empty((batch, cfg.groups, max(cfg.topk, 1)), dtype=torch.int32, device=q.device)
    cnt = torch.empty((batch, cfg.groups), dtype=torch.int32, device=q.device)
    if ws is None:
        ws = step_workspace(cfg, batch, mb, q.device)
    B.kvs_decode_step(cfg, q, k_pool, v_pool, rep_pool, block_table, mb, seq_lens, batch, out,
                      sel, cnt, ws, ws.numel())
    return out, sel[:, :, : cfg.topk], cnt
