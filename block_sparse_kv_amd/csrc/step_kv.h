// Launchers of the decode step's kernels, one instantiation per kv_type (step_fp16.hip, step_q8.hip,
// step_q4.hip, step_i8.hip), so the four compile in parallel.
#pragma once

#include "kvs_launch.h"

namespace kvs {

constexpr int kStepTopkKeys = 8;  // keys per lane of the 256-lane selections
constexpr int kStepTopkSmall = 256 * kStepTopkKeys;  // rows up to this many blocks: one fused launch

// Chunk summaries of the long-row selection: [batch][G][chunks][8] scores, block ids and physical ids
// (all null for the register selection over whole rows).
struct Summaries {
  float* val = nullptr;
  int32_t* id = nullptr;
  int32_t* phys = nullptr;
};

// Rows of SEPARATE selections up to this many blocks take the fused launch through chunk summaries
// (8 summary entries per 64-block chunk, at most 8 per lane of the 256-lane selection).
constexpr int kStepSummMax = 256 * 8 * 8;

// The selected tiles' workgroups make their groups' selections themselves while they number at most
// this many (batch * num_kv_heads * topk): all of them resident at once.
constexpr int kSelByTilesMax = 1024;

// Scoring, the top-k by the group's last scoring workgroup (sel != nullptr) and the Initial/Local tiles
// [0, il_per) of each KV head (every one for il_per < 0), in one launch: rows of up to kStepTopkSmall
// blocks from the whole score row, longer SEPARATE rows (up to kStepSummMax) from the chunk
// summaries U.
template <int KV>
hipError_t launch_score_select_kv(const AttnArgs& A, const void* rep_pool, float* scores, int32_t* sel,
                                  int32_t* cnt, int32_t* tiles, int* ctr, int batch, hipStream_t s,
                                  const Summaries& U, int il_per = -1);
// The selected tiles, and the Initial/Local tiles [il0, n_il_max) of each KV head, of a step whose
// rows (up to kStepTopkSmall blocks) were scored by an earlier launch into scores: each selected
// tile's workgroup makes its group's selection itself.
// With U (SEPARATE rows of up to kStepSummMax blocks, topk <= kSummSlotMax), from the chunk summaries
// the scoring launch stored; with n_list > 0, from the preselected sets U.id [rows][n_list] (at most
// kPreselStepMax entries) and their scores and physical ids U.val / U.phys stored by the scoring.
template <int KV>
hipError_t launch_attn_select_kv(const AttnArgs& A, const float* scores, int32_t* sel, int32_t* sel_count,
                                 int batch, int il0, hipStream_t s, const Summaries& U, int n_list = 0);
// Longer rows: the top-k selections (512-lane workgroups) and the Initial/Local tiles in one launch.
template <int KV>
hipError_t launch_topk_il_wide_kv(const AttnArgs& A, const float* scores, int32_t* sel, int32_t* sel_count,
                                  int32_t* tiles, int batch, hipStream_t s);

// The confined step's first launch: scoring of the preselected sets, the selection from them and the
// Initial/Local tiles (sets of up to kPreselStepMax entries; 256-lane selection, kPreselStepKeys keys
// per lane).
constexpr int kPreselStepKeys = 4;
constexpr int kPreselStepMax = 256 * kPreselStepKeys;
// With sel null: the scoring only (and the Initial/Local tiles [0, il_per) of each KV head; every one
// for il_per < 0).
template <int KV>
hipError_t launch_presel_step_kv(const AttnArgs& A, const void* rep_pool, const int32_t* presel,
                                 int n_presel, float* cs, int32_t* cph, int32_t* sel, int32_t* cnt,
                                 int32_t* tiles, int* ctr, int batch, hipStream_t s, int il_per = -1);

}  // namespace kvs
