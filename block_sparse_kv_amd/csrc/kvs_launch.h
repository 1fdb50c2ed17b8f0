// Internal launchers of libkvs (host side).  Arguments are validated by kvs_api.cpp before any of
// these is called; each enqueues on `s` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvs_device.h"

namespace kvs {

// Split plan of the attention kernel: `tps` tiles per workgroup, `n_splits` workgroups per
// (sequence, KV head), and the workspace the partials need.  A pure function of the config and
// sizes, so the size query and the launch always agree.
struct AttnPlan {
  int maxT;      // upper bound on attended tiles per (sequence, group)
  int tps, n_splits;
  size_t part_o_bytes, part_ml_bytes, tiles_bytes, ntiles_bytes;
};
AttnPlan attn_plan(const Params& P, int batch, int max_blocks);

hipError_t launch_build_reps(const Params& P, const void* k_pool, const int32_t* ids, int n,
                             int rep_num, void* rep_pool, hipStream_t s);
hipError_t launch_score(const Params& P, const void* q, const void* rep_pool, const int32_t* table,
                        int max_blocks, const int32_t* seq_lens, int batch, float* scores,
                        hipStream_t s);
hipError_t launch_topk(const Params& P, const float* scores, const int32_t* seq_lens, int batch,
                       int max_blocks, int32_t* sel, int32_t* sel_count, hipStream_t s);
// Physical tile list of every (sequence, group): tiles [batch][G][maxT] (-1 padded), ntiles [batch][G].
hipError_t launch_tile_plan(const Params& P, const AttnPlan& A, const int32_t* table, int max_blocks,
                            const int32_t* seq_lens, int batch, const int32_t* sel,
                            const int32_t* sel_count, int32_t* tiles, int32_t* ntiles, hipStream_t s);
// Split attention over a tile list, then the log-sum-exp merge into out.
hipError_t launch_attn(const Params& P, const AttnPlan& A, const void* q, const void* k_pool,
                       const void* v_pool, const int32_t* seq_lens, int batch, const int32_t* tiles,
                       const int32_t* ntiles, float* out, float* part_o, float* part_ml,
                       hipStream_t s);

// ---- fused decode step (step.hip) -------------------------------------------------------------
constexpr int kCtrlHead = 64;  // ints before the per-sequence counters: [0] ticket, [1] exit, [2] error

// Work decomposition of one kvs_decode_step call; a pure function of config, sizes and the number of
// resident workgroups.
struct StepPlan {
  int sb, n_score_per_seq;          // blocks per score item, score items per sequence
  int tps_il, n_il_parts;           // Initial/Local tiles per item, items per (sequence, KV head)
  int tps_sel, n_sel_parts;         // selected tiles per item, items per (sequence, KV head)
  int n_parts;                      // partials per (sequence, KV head)
  int off_topk, off_il, off_sel, total;  // ticket ranges of the item kinds
  int ctrl_ints;
  size_t part_o_bytes, part_ml_bytes, tiles_bytes;
};
StepPlan step_plan(const Params& P, int batch, int max_blocks, int resident_wgs);

struct StepArgs {
  Params P;
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const void* rep_pool;
  const int32_t* table;
  const int32_t* seq_lens;
  float* out;
  int32_t* sel;        // [batch][G][topk]
  int32_t* sel_count;  // [batch][G]
  float* scores;       // [batch][G][max_blocks]
  int32_t* tiles_sel;  // [batch][G][topk] physical ids of the selected tiles
  float* part_o;       // [batch][Hq][n_parts][128]
  float* part_ml;      // [batch][Hq][n_parts][2]
  int* ctrl;           // zero before the call; zero again after it
  int max_blocks, batch;
  int sb, n_score_per_seq, tps_il, n_il_parts, tps_sel, n_sel_parts, n_parts;
  int off_topk, off_il, off_sel, total;
};

hipError_t step_resident_wgs(const Params& P, int* out);
hipError_t launch_step(const StepArgs& A, int grid, hipStream_t s);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace kvs
