// Launchers of the decode step's kernels, one instantiation per kv_type (step_fp16.hip, step_q8.hip,
// step_q4.hip, step_i8.hip), so the four compile in parallel.
#pragma once

#include "kvs_launch.h"

namespace kvs {

constexpr int kStepTopkKeys = 8;  // keys per lane of the 256-lane selections
constexpr int kStepTopkSmall = 256 * kStepTopkKeys;  // rows up to this many blocks: one fused launch

// Scoring, the top-k by the group's last scoring workgroup (sel != nullptr) and the Initial/Local tiles,
// in one launch (rows of up to kStepTopkSmall blocks).
template <int KV>
hipError_t launch_score_select_kv(const AttnArgs& A, const void* rep_pool, float* scores, int32_t* sel,
                                  int32_t* cnt, int32_t* tiles, int* ctr, int batch, hipStream_t s);
// Longer rows: the top-k selections (512-lane workgroups) and the Initial/Local tiles in one launch.
template <int KV>
hipError_t launch_topk_il_wide_kv(const AttnArgs& A, const float* scores, int32_t* sel, int32_t* sel_count,
                                  int32_t* tiles, int batch, hipStream_t s);

}  // namespace kvs
