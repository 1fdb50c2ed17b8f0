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
  int tps, n_splits;
  size_t part_o_bytes, part_ml_bytes;
};
AttnPlan attn_plan(const Params& P, int batch, int max_blocks);

hipError_t launch_build_reps(const Params& P, const void* k_pool, const int32_t* ids, int n,
                             int rep_num, void* rep_pool, hipStream_t s);
hipError_t launch_score(const Params& P, const void* q, const void* rep_pool, const int32_t* table,
                        int max_blocks, const int32_t* seq_lens, int batch, float* scores,
                        hipStream_t s);
hipError_t launch_topk(const Params& P, const float* scores, const int32_t* seq_lens, int batch,
                       int max_blocks, int32_t* sel, int32_t* sel_count, hipStream_t s);
hipError_t launch_attn(const Params& P, const AttnPlan& A, const void* q, const void* k_pool,
                       const void* v_pool, const int32_t* table, int max_blocks,
                       const int32_t* seq_lens, int batch, const int32_t* sel,
                       const int32_t* sel_count, float* out, float* part_o, float* part_ml,
                       hipStream_t s);

}  // namespace kvs
