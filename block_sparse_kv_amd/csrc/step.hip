// kvs_decode_step: scoring -> top-k -> attention tiles -> merge, with the Initial/Local tiles -- which
// do not depend on the selection [KT-LC §4.2] -- placed where their K/V gather costs least:
//  * short rows (max_blocks <= kStepTopkSmall) of small batches (select_plan): a scoring launch
//    (score_select_kernel without its selection), with some of the Initial/Local tiles; then one
//    launch in which every selected tile's workgroup makes its group's selection from the score row
//    itself (all of them make the same one) and gathers its own entry, beside the other Initial/Local
//    tiles (attn_select_kernel); then the merge (attn.hip).
//  * other short rows: one launch scores, selects and gathers the Initial/Local tiles
//    (score_select_kernel).  The scoring workgroups of a (sequence, group) hand their scores to the
//    one among them that finishes last, which makes the group's selection (256 lanes, keys in
//    registers); the Initial/Local tiles stream meanwhile.  Then the selected tiles and the merge.
//  * SEPARATE rows of up to kStepSummMax blocks: each scoring workgroup (one 64-block chunk of one KV
//    head) also stores its chunk's best 8, and the selection is made from these summaries, or from
//    the whole row when a chunk holds more than 8 of the selection -- for small batches by every
//    selected tile's workgroup, as for the short rows above (all Initial/Local tiles in the tiles'
//    launch), else by the last scoring workgroup of the KV head in the scoring launch.
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
                               const Summaries& U = Summaries(), int il_per = -1) {
  switch (A.P.kv) {
    case kKvQ8: return launch_score_select_kv<kKvQ8>(A, rep_pool, scores, sel, cnt, tiles, ctr, batch, s, U, il_per);
    case kKvQ4: return launch_score_select_kv<kKvQ4>(A, rep_pool, scores, sel, cnt, tiles, ctr, batch, s, U, il_per);
    case kKvI8: return launch_score_select_kv<kKvI8>(A, rep_pool, scores, sel, cnt, tiles, ctr, batch, s, U, il_per);
    case kKvI4: return launch_score_select_kv<kKvI4>(A, rep_pool, scores, sel, cnt, tiles, ctr, batch, s, U, il_per);
    default: return launch_score_select_kv<kKvFp16>(A, rep_pool, scores, sel, cnt, tiles, ctr, batch, s, U, il_per);
  }
}

hipError_t launch_attn_select(const AttnArgs& A, const float* scores, int32_t* sel, int32_t* sel_count, int batch,
                              int il0, hipStream_t s, const Summaries& U, int n_list = 0) {
  switch (A.P.kv) {
    case kKvQ8: return launch_attn_select_kv<kKvQ8>(A, scores, sel, sel_count, batch, il0, s, U, n_list);
    case kKvQ4: return launch_attn_select_kv<kKvQ4>(A, scores, sel, sel_count, batch, il0, s, U, n_list);
    case kKvI8: return launch_attn_select_kv<kKvI8>(A, scores, sel, sel_count, batch, il0, s, U, n_list);
    case kKvI4: return launch_attn_select_kv<kKvI4>(A, scores, sel, sel_count, batch, il0, s, U, n_list);
    default: return launch_attn_select_kv<kKvFp16>(A, scores, sel, sel_count, batch, il0, s, U, n_list);
  }
}

// Rows of up to kStepTopkSmall blocks: whether every selected tile's workgroup makes its group's
// selection itself (by_tiles) rather than the scoring launch's last workgroup of the group, and how
// many of each KV head's Initial/Local tiles stream in the scoring launch (il_first; the rest stream
// in the tiles' launch while the selections are made).  Chosen by measurement:
//  * by_tiles while the selected tiles' workgroups number at most kSelByTilesMax, all resident at
//    once; with more (large batches) the same selections would be made over several waves of
//    workgroups, and the last scoring workgroup of each group makes each once instead (16 sequences
//    of 16K to 128K tokens: 109 against 121 us per step);
//  * rows of up to 256 blocks: up to kIlLate Initial/Local tiles per KV head stream beside the
//    selections, the others beside the scoring (32K tokens, 8 KV heads: 19.4 us per step, against
//    20.8 with all of them beside the selections and 20.1 with all beside the scoring); longer rows:
//    all beside the selections (128K tokens: 23.9 us, against 24.5 with half beside the scoring).
// SEPARATE rows of up to kStepSummMax blocks select from chunk summaries (summ): the scoring launch
// stores them, and the selected tiles' workgroups select from them the same way, with every
// Initial/Local tile beside the selections (1M tokens, 8 KV heads, k 64: 906 against 952 us per step
// of 32 layers, where the scoring launch's last workgroups selected and the tiles streamed beside).
constexpr int kIlLate = 16;
struct SelPlan {
  bool by_tiles, summ;
  int il_first;
};
SelPlan select_plan(const Params& P, int batch, int max_blocks, int n_il_max, bool summ) {
  SelPlan p{false, false, n_il_max};
  if (P.topk <= 0 || (long long)batch * P.Hkv * P.topk > kSelByTilesMax) return p;
  if (max_blocks <= kStepTopkSmall) {
    p.by_tiles = true;
    p.il_first = max_blocks <= 256 ? (n_il_max > kIlLate ? n_il_max - kIlLate : 0) : 0;
  } else if (summ) {
    p.by_tiles = p.summ = true;
    p.il_first = 0;
  }
  return p;
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

// The confined step's scoring and tiles: as for the decode step's short rows (select_plan), while the
// selected tiles' workgroups number at most kSelByTilesMax each makes its row's selection from the
// scored set itself, with up to kIlLate Initial/Local tiles per KV head beside the selections for sets
// of up to 256 entries (every one beside them for larger sets); otherwise the scoring launch's last
// workgroup of each row selects, and the selected tiles follow in a launch of their own.
hipError_t launch_presel_step(const AttnArgs& A, const void* rep_pool, const int32_t* presel, int n_presel,
                              float* cs, int32_t* cph, int32_t* sel, int32_t* cnt, int32_t* tiles, int* ctr,
                              int batch, hipStream_t s) {
  const bool by_tiles = (long long)batch * A.P.Hkv * A.P.topk <= kSelByTilesMax;
  const int il_per = !by_tiles ? -1 : n_presel <= 256 ? (A.n_il_max > kIlLate ? A.n_il_max - kIlLate : 0) : 0;
  int32_t* ssel = by_tiles ? nullptr : sel;
  hipError_t e;
#define KVS_PS_ONE(KK) \
  launch_presel_step_kv<KK>(A, rep_pool, presel, n_presel, cs, cph, ssel, cnt, tiles, ctr, batch, s, il_per)
  switch (A.P.kv) {
    case kKvQ8: e = KVS_PS_ONE(kKvQ8); break;
    case kKvQ4: e = KVS_PS_ONE(kKvQ4); break;
    case kKvI8: e = KVS_PS_ONE(kKvI8); break;
    case kKvI4: e = KVS_PS_ONE(kKvI4); break;
    default: e = KVS_PS_ONE(kKvFp16); break;
  }
#undef KVS_PS_ONE
  if (e != hipSuccess) return e;
  if (!by_tiles) return launch_attn_tiles(A, batch, false, true, s);
  Summaries L;  // the sets, their scores and physical ids by position
  L.val = cs;
  L.id = const_cast<int32_t*>(presel);
  L.phys = cph;
  return launch_attn_select(A, cs, sel, cnt, batch, il_per, s, L, n_presel);
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
  Summaries U;
  if (ub != 0 && summ != nullptr) {
    U.val = static_cast<float*>(summ);
    U.id = reinterpret_cast<int32_t*>(static_cast<char*>(summ) + ub);
    U.phys = reinterpret_cast<int32_t*>(static_cast<char*>(summ) + 2 * ub);
  }
  const SelPlan sp = select_plan(P, batch, A.max_blocks, A.n_il_max, U.val != nullptr);
  if (sp.by_tiles) {
    const Summaries Us = sp.summ ? U : Summaries();
    e = launch_score_select(A, rep_pool, scores, nullptr, nullptr, nullptr, nullptr, batch, s, Us, sp.il_first);
    if (e == hipSuccess) e = launch_attn_select(A, scores, sel, sel_count, batch, sp.il_first, s, Us);
  } else if (A.max_blocks <= kStepTopkSmall) {
    e = launch_score_select(A, rep_pool, scores, sel, sel_count, tl, ctr, batch, s);
    if (e == hipSuccess) e = launch_attn_tiles(A, batch, false, true, s);
  } else if (U.val != nullptr && P.topk > 0) {  // one launch scores and selects
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
