// Internal launchers of libkvs (host side).  Arguments are validated by kvs_api.cpp before any of
// these is called; each enqueues on `s` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvs_device.h"

namespace kvs {

// Partials of the attention: per (sequence, query head) at most max_parts = n_il_max + topk, where
// n_il_max bounds the Initial + Local tiles of any sequence.  A pure function of the config and sizes,
// so the workspace query and the launch always agree.
struct AttnPlan {
  int n_il_max, max_parts;
  size_t part_o_bytes, part_ml_bytes;
};
AttnPlan attn_plan(const Params& P, int batch, int max_blocks);

hipError_t launch_quantize_q8(const Params& P, const void* src, const int32_t* ids, int n, void* dst,
                              hipStream_t s);
hipError_t launch_token_importance(const Params& P, const void* q_obs, int n_obs, const void* k_pool,
                                   const int32_t* table, int max_blocks, const int32_t* seq_lens, int batch,
                                   float* imp, void* ws, hipStream_t s);
size_t token_importance_ws_bytes(const Params& P, int batch, int max_blocks, int n_obs);
hipError_t launch_dynamic_reps(const Params& P, const void* k_pool, const float* imp, const int32_t* table,
                               int max_blocks, const int32_t* seq_lens, int batch, void* rep_pool,
                               hipStream_t s);
// pool_kernel 0: block sums; odd 1..127: best pooled vote per block.
hipError_t launch_block_scores(const Params& P, const float* imp, const int32_t* seq_lens, int batch,
                               int max_blocks, int pool_kernel, float* bs, hipStream_t s);
hipError_t launch_presel_select(const Params& P, const float* scores, int max_blocks, const int32_t* seq_lens,
                                const int32_t* presel, int n_presel, int batch, int32_t* sel,
                                int32_t* sel_count, hipStream_t s);
hipError_t launch_compact(const Params& P, const float* scores, int max_blocks, const int32_t* seq_lens,
                          const int32_t* presel, int n_presel, int batch, float* cs, int32_t* cid,
                          int32_t* clen, hipStream_t s);
hipError_t launch_map_back(const int32_t* csel, int topk, const int32_t* cid, int n_presel, int rows,
                           int32_t* sel, hipStream_t s);
hipError_t launch_build_reps(const Params& P, const void* k_pool, const int32_t* ids, int n,
                             int rep_num, void* rep_pool, hipStream_t s);
hipError_t launch_score(const Params& P, const void* q, const void* rep_pool, const int32_t* table,
                        int max_blocks, const int32_t* seq_lens, int batch, float* scores,
                        hipStream_t s);
// table / tiles nullable: with both, tiles [batch][G][topk] receives the physical ids of the
// selection (-1 padded).
hipError_t launch_topk(const Params& P, const float* scores, const int32_t* seq_lens, int batch,
                       int max_blocks, int32_t* sel, int32_t* sel_count, const int32_t* table,
                       int32_t* tiles, hipStream_t s);
// Attention work items: with il, the Initial/Local tiles and then the selected ones, else only the
// selected ones; A.sel holds physical ids if sel_phys, logical ids otherwise.
hipError_t launch_attn_tiles(const AttnArgs& A, int batch, bool il, bool sel_phys, hipStream_t s);
hipError_t launch_merge(const AttnArgs& A, int batch, hipStream_t s);
// The read floor of the tile gather (measurement): n tiles phys * Hkv + h of the fp16 pools (ids
// outside [0, pool_tiles) give NaN), each summed into out[x]; lds_bytes of LDS reserved per workgroup.
hipError_t launch_gather_read(const void* k_pool, const void* v_pool, int pool_tiles, const int32_t* ids,
                              int n, int lds_bytes, float* out, hipStream_t s);
// Hand-off counters of the decode step: kStepCtrBytes of ints, one per (sequence, group) at index
// (seq * G + group) * step_ctr_stride(batch * G), so that counters fall on separate 128-byte lines as
// far as they fit (agent-scope atomics on one line are serialized where memory performs them).
constexpr size_t kStepCtrBytes = 65536;
inline int step_ctr_stride(int n_ctr) {
  int st = 32;
  while (st > 1 && (size_t)n_ctr * st * sizeof(int) > kStepCtrBytes) st >>= 1;
  return st;
}
// The whole decode step (step.hip): scores [batch][G][max_blocks], sel / sel_count, and the selected
// tiles' physical ids (tiles [batch][G][topk]) are its intermediates; A.sel must be `tiles`.  ctr:
// the kStepCtrBytes counter area, zero when the call starts and zero again when it ends.
// Scores [batch][G][max_blocks] of every candidate, and, for rows the fused step handles in one
// launch (max_blocks <= 2048), the Initial/Local tiles in the same launch (*il_done = true).
hipError_t launch_score_il(const AttnArgs& A, const void* rep_pool, float* scores, int batch, hipStream_t s,
                           bool* il_done);
// summ: the chunk summaries of the long-row selection, three arrays of summaries_bytes() each (val,
// id, phys), nullable (then long rows take the separate top-k launch).
size_t summaries_bytes(const Params& P, int batch, int max_blocks);
hipError_t launch_decode_step(const AttnArgs& A, const void* rep_pool, float* scores, int32_t* sel,
                              int32_t* sel_count, int32_t* tiles, int* ctr, int batch, hipStream_t s,
                              void* summ);

// The confined step up to its merge (step.hip): the sets presel [batch][G][n_presel] (n_presel <=
// presel_step_max()) scored into cs / cph [batch][G][n_presel] (scores, physical ids), the selection
// (sel: logical ids, cnt; tiles: physical ids, when the scoring launch makes it), and the attention
// over the Initial/Local and selected tiles into A's partials; ctr as for launch_decode_step.
int presel_step_max();
hipError_t launch_presel_step(const AttnArgs& A, const void* rep_pool, const int32_t* presel, int n_presel,
                              float* cs, int32_t* cph, int32_t* sel, int32_t* cnt, int32_t* tiles, int* ctr,
                              int batch, hipStream_t s);

}  // namespace kvs
