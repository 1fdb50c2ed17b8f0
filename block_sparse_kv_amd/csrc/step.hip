// kvs_decode_step: scoring -> top-k -> attention tiles -> merge, with the Initial/Local tiles -- which
// do not depend on the selection [KT-LC §4.2] -- placed where their K/V gather costs least:
//  * short rows (max_blocks <= kStepTopkSmall): one launch scores, selects and gathers the
//    Initial/Local tiles (score_select_kernel).  The scoring workgroups of a (sequence, group) hand
//    their scores to the one among them that finishes last, which makes the group's selection (256
//    lanes, keys in registers); the Initial/Local tiles stream meanwhile.  Then the selected tiles
//    and the merge (attn.hip).
//  * SEPARATE rows of up to kStepSummMax blocks: the same launch, each scoring workgroup (one 64-block
//    chunk of one KV head) also storing its chunk's best 8; the last one selects from these summaries,
//    or from the whole row when a chunk holds more than 8 of the selection.
//  * other long rows: scoring (score.hip); then the top-k selections in 512-lane workgroups with the
//    Initial/Local tiles, two per workgroup, in one launch (topk_il_wide_kernel), so their gather
//    runs while the selections are made; then the selected tiles and the merge.
// The confined step (kvs_decode_step_preselected) scores only the preselected sets and selects from
// them in the same way (presel_step_kernel), then runs the selected tiles and the merge.
// In every grid an attention tile is one workgroup (attn_core.h).
#include "kvs_launch.h"
#include "step_kv.h"

namespace kvs {

namespace {
hipError_t launch_score_select(const AttnArgs& A, const void* rep_pool, float* scores, int32_t* sel,
                               int32_t* cnt, int32_t* tiles, int* ctr, int batch, hipStream_t s,
                               const Summaries& U = Summaries()) {
  switch (A.P.kv) {
    case kKvQ8: return launch_score_select_kv<kKvQ8>(A, rep_pool, scores, sel, cnt, tiles, ctr, batch, s, U);
    case kKvQ4: return launch_score_select_kv<kKvQ4>(A, rep_pool, scores, sel, cnt, tiles, ctr, batch, s, U);
    case kKvI8: return launch_score_select_kv<kKvI8>(A, rep_pool, scores, sel, cnt, tiles, ctr, batch, s, U);
    case kKvI4: return launch_score_select_kv<kKvI4>(A, rep_pool, scores, sel, cnt, tiles, ctr, batch, s, U);
    default: return launch_score_select_kv<kKvFp16>(A, rep_pool, scores, sel, cnt, tiles, ctr, batch, s, U);
  }
}

hipError_t launch_topk_il_wide(const AttnArgs& A, const float* scores, int32_t* sel, int32_t* sel_count,
                               int32_t* tiles, int batch, hipStream_t s) {
  switch (A.P.kv) {
    case kKvQ8: return launch_topk_il_wide_kv<kKvQ8>(A, scores, sel, sel_count, tiles, batch, s);
    case kKvQ4: return launch_topk_il_wide_kv<kKvQ4>(A, scores, sel, sel_count, tiles, batch, s);
    case kKvI8: return launch_topk_il_wide_kv<kKvI8>(A, scores, sel, sel_count, tiles, batch, s);
    case kKvI4: return launch_topk_il_wide_kv<kKvI4>(A, scores, sel, sel_count, tiles, batch, s);
    default: return launch_topk_il_wide_kv<kKvFp16>(A, scores, sel, sel_count, tiles, batch, s);
  }
}
}  // namespace

hipError_t launch_score_il(const AttnArgs& A, const void* rep_pool, float* scores, int batch, hipStream_t s,
                           bool* il_done) {
  *il_done = A.max_blocks <= kStepTopkSmall;
  if (*il_done) return launch_score_select(A, rep_pool, scores, nullptr, nullptr, nullptr, nullptr, batch, s);
  return launch_score(A.P, A.q, rep_pool, A.table, A.max_blocks, A.seq_lens, batch, scores, s);
}

int presel_step_max() { return kPreselStepMax; }

hipError_t launch_presel_step(const AttnArgs& A, const void* rep_pool, const int32_t* presel, int n_presel,
                              float* cs, int32_t* cph, int32_t* sel, int32_t* cnt, int32_t* tiles, int* ctr,
                              int batch, hipStream_t s) {
  switch (A.P.kv) {
    case kKvQ8: return launch_presel_step_kv<kKvQ8>(A, rep_pool, presel, n_presel, cs, cph, sel, cnt, tiles, ctr, batch, s);
    case kKvQ4: return launch_presel_step_kv<kKvQ4>(A, rep_pool, presel, n_presel, cs, cph, sel, cnt, tiles, ctr, batch, s);
    case kKvI8: return launch_presel_step_kv<kKvI8>(A, rep_pool, presel, n_presel, cs, cph, sel, cnt, tiles, ctr, batch, s);
    case kKvI4: return launch_presel_step_kv<kKvI4>(A, rep_pool, presel, n_presel, cs, cph, sel, cnt, tiles, ctr, batch, s);
    default: return launch_presel_step_kv<kKvFp16>(A, rep_pool, presel, n_presel, cs, cph, sel, cnt, tiles, ctr, batch, s);
  }
}

size_t summaries_bytes(const Params& P, int batch, int max_blocks) {
  if (!(P.mode == kSeparate && max_blocks > kStepTopkSmall && max_blocks <= kStepSummMax)) return 0;
  return (size_t)batch * P.G * ((max_blocks + kChunkBlocks - 1) / kChunkBlocks) * kChunkTop * 4;
}

hipError_t launch_decode_step(const AttnArgs& A, const void* rep_pool, float* scores, int32_t* sel,
                              int32_t* sel_count, int32_t* tiles, int* ctr, int batch, hipStream_t s,
                              void* summ) {
  const Params& P = A.P;
  int32_t* tl = P.topk > 0 ? tiles : nullptr;
  hipError_t e;
  const size_t ub = summaries_bytes(P, batch, A.max_blocks);
  if (A.max_blocks <= kStepTopkSmall) {
    e = launch_score_select(A, rep_pool, scores, sel, sel_count, tl, ctr, batch, s);
    if (e == hipSuccess) e = launch_attn_tiles(A, batch, false, true, s);
  } else if (ub != 0 && summ != nullptr && P.topk > 0) {  // one launch scores and selects
    Summaries U;
    U.val = static_cast<float*>(summ);
    U.id = reinterpret_cast<int32_t*>(static_cast<char*>(summ) + ub);
    U.phys = reinterpret_cast<int32_t*>(static_cast<char*>(summ) + 2 * ub);
    e = launch_score_select(A, rep_pool, scores, sel, sel_count, tl, ctr, batch, s, U);
    if (e == hipSuccess) e = launch_attn_tiles(A, batch, false, true, s);
  } else {
    e = launch_score(P, A.q, rep_pool, A.table, A.max_blocks, A.seq_lens, batch, scores, s);
    if (e == hipSuccess) e = launch_topk_il_wide(A, scores, sel, sel_count, tl, batch, s);
    if (e == hipSuccess) e = launch_attn_tiles(A, batch, false, true, s);
  }
  if (e == hipSuccess) e = launch_merge(A, batch, s);
  return e;
}

}  // namespace kvs
