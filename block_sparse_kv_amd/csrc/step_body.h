// Kernels of kvs_decode_step (their dispatch over the cache type is step.hip's): compiled once per
// kv_type by the step_*.hip files, each instantiating the launchers for its own type.
#pragma once

#include "attn_core.h"
#include "kvs_launch.h"
#include "step_kv.h"
#include "score_core.h"
#include "topk_core.h"

namespace kvs {

constexpr int kStepLds = kAttnLdsBytes > (int)sizeof(TopkLds) ? kAttnLdsBytes : (int)sizeof(TopkLds);
// attn_select_kernel, kSrcSumm: where a whole-row selection (topk entries, then their physical ids) goes in
// LDS, after the selection's own TopkLds; kSummSlotMax entries fit.
constexpr int kSummSlotOff = ((int)sizeof(TopkLds) + 15) / 16 * 16;
constexpr int kSummSlotMax = (kStepLds - kSummSlotOff) / 8;
static_assert(kSummSlotMax >= kSelByTilesMax, "every topk the in-tile selections take fits");

// The chunk summary of one SEPARATE scoring workgroup (called by all 256 lanes; chunk = its
// kChunkBlocks blocks, whose scores are in lds[0..kChunkBlocks) and physical ids in lds[kChunkBlocks..)
// as ints): the kChunkTop best by (score desc, block asc), written by wave 0 sorted by block, padded
// with (-inf, -1, 0), coherently to u*[chunk * kChunkTop ..].  Block b0 + i is lane i of each wave;
// each wave counts the blocks among its 16 of the chunk that come before lane i's (all four waves
// share the comparisons, so that no one SIMD carries them), the counts meet in LDS after the
// chunk's ids (lds[2 * kChunkBlocks ..], 4 x 64 ints), and wave 0 adds them.  Waves 1..3 return
// after the barrier.
__device__ inline void write_chunk_summary(const float* lds, int b0, float* uval, int32_t* uid,
                                           int32_t* uphys) {
  static_assert(kChunkBlocks == 64, "one block per lane");
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const float v = lds[lane];
  int* prank = reinterpret_cast<int*>(const_cast<float*>(lds)) + 2 * kChunkBlocks;  // [wave][block]
  {
    int r = 0;
#pragma unroll
    for (int jj = 0; jj < 16; jj += 4) {
      const int j = 16 * wv + jj;
      const float4 q = *reinterpret_cast<const float4*>(lds + j);
      r += (q.x > v || (q.x == v && j < lane)) ? 1 : 0;
      r += (q.y > v || (q.y == v && j + 1 < lane)) ? 1 : 0;
      r += (q.z > v || (q.z == v && j + 2 < lane)) ? 1 : 0;
      r += (q.w > v || (q.w == v && j + 3 < lane)) ? 1 : 0;
    }
    prank[wv * 64 + lane] = r;
  }
  __syncthreads();
  if (wv != 0) return;
  const int phys = reinterpret_cast<const int*>(lds)[kChunkBlocks + lane];
  const int rank = (prank[lane] + prank[64 + lane]) + (prank[128 + lane] + prank[192 + lane]);
  // the taken blocks (the first kChunkTop by rank that are candidates) in block order, then padding
  const bool take = rank < kChunkTop && v > -INFINITY;
  const unsigned long long tk = __ballot(take);
  const int n_take = __popcll(tk);
  const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(tk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)tk, 0));
  if (take) {
    st_coh(uval + pos, v);
    st_coh(uid + pos, b0 + lane);
    st_coh(uphys + pos, phys);
  }
  if (lane >= n_take && lane < kChunkTop) {
    st_coh(uval + lane, -INFINITY);
    st_coh(uid + lane, -1);
    st_coh(uphys + lane, 0);
  }
}

// First the scoring workgroups, n_sc per (sequence, group), over every KV head (SHARED) or over one KV
// head (SEPARATE; group = KV head): dispatched first, their few loads are not queued behind the
// tiles' stream.  With sel null the kernel only scores (and, SUMM, stores the chunk summaries) and
// streams the tiles (the selections are made by later launches).  Then n_il_wg Initial/Local tiles, il_per (<= n_il_max) per KV head: tile t < il_per
// of KV head h of sequence seq at (seq * Hkv + h) * il_per + t.  A scoring workgroup stores its
// scores coherently, waits for them to complete and bumps the group's counter; the one that brings it
// to n_sc resets it and selects.  Nothing waits on another workgroup.
// SUMM (SEPARATE rows longer than the register selection holds): each scoring workgroup, one chunk of
// kChunkBlocks blocks, also writes its chunk summary; the last one selects from the summaries
// (topk_summary_reg) and, if a chunk holds more than kChunkTop of the selection, from the whole row.
template <int G, int METHOD, int MODE, int KV, bool SUMM = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 4 : 2))) void score_select_kernel(
    AttnArgs A, const void* __restrict__ rep_pool, float* __restrict__ scores, int32_t* __restrict__ sel,
    int32_t* __restrict__ sel_count, int32_t* __restrict__ tiles, int* __restrict__ ctr, int ctr_stride,
    int n_sc, int n_il_wg, int il_per, float* __restrict__ uval, int32_t* __restrict__ uid,
    int32_t* __restrict__ uphys) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStepLds];
  __shared__ int s_last;
  const Params& P = A.P;
  const int n_score_wg = (int)gridDim.x - n_il_wg;
  const int x = blockIdx.x;
  if (x >= n_score_wg) {
    const int xi = x - n_score_wg;
    const int per_seq = P.Hkv * il_per;
    const int r = xi % per_seq;
    attn_item<G, true, false, KV>(A, r % il_per, r / il_per, xi / per_seq, smem);
    return;
  }
  constexpr bool SEP = MODE == kSeparate;
  KVS_TL_BEGIN(P, kTlScoreSel, 256)
  const int y = x;
  const int per_seq = P.G * n_sc;
  const int seq = y / per_seq, grp = (y % per_seq) / n_sc, c = y % n_sc;
  const int sb = SEP ? kScoreBlocksPerHeadWg : score_blocks_per_wg(P);
  static_assert(kScoreBlocksPerHeadWg == kChunkBlocks, "a SEPARATE scoring workgroup is one chunk");
  const int32_t* trow = A.table + (size_t)seq * A.max_blocks;
  float* lchunk = reinterpret_cast<float*>(smem) + 64;  // SEPARATE scoring leaves the first floats unused
  score_blocks_range<G, METHOD, MODE, SEP, true>(P, A.q + (size_t)seq * P.Hq * kDim, rep_pool, trow,
                                                 A.max_blocks, A.seq_lens[seq], c * sb, sb,
                                                 scores + (size_t)seq * P.G * A.max_blocks,
                                                 reinterpret_cast<float*>(smem), grp, SUMM ? lchunk : nullptr);
  KVS_TL_MARK_LOADED(1)
  if (!SUMM && sel == nullptr) return;  // scores and Initial/Local tiles only: the selection comes later
  const size_t urow = ((size_t)seq * P.G + grp) * n_sc * kChunkTop;  // this group's summaries
  if constexpr (SUMM) {
    __syncthreads();  // the chunk's scores are in LDS
    write_chunk_summary(lchunk, c * sb, uval + urow + (size_t)c * kChunkTop,
                        uid + urow + (size_t)c * kChunkTop, uphys + urow + (size_t)c * kChunkTop);
    KVS_TL_MARK(5)
    if (sel == nullptr) return;  // scores and summaries only: the selections come later
  }
  wait_mem();
  if constexpr (SUMM) {
    KVS_TL_MARK(4)
  }
  __syncthreads();
  int* cp = ctr + ((size_t)seq * P.G + grp) * ctr_stride;
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(cp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n_sc - 1;
  __syncthreads();
  KVS_TL_MARK(2)
  if (!s_last) return;  // else every scoring workgroup of the group has arrived
  if constexpr (SUMM) {
    const size_t row = (size_t)seq * P.G + grp;
    const Regions rg = regions_of(A.seq_lens[seq], P.initial_len, P.local_len);
    const int cand_hi = min(rg.cand_hi, A.max_blocks);
    const int n = max(0, cand_hi - rg.cand_lo);
    const int k = min(P.topk, n);
    int32_t* out = sel + row * P.topk;
    int32_t* tout = tiles ? tiles + row * P.topk : nullptr;
    TopkLds& S = *reinterpret_cast<TopkLds*>(smem);
    if (k >= n) {  // every candidate (or none)
      for (int i = threadIdx.x; i < n; i += 256) {
        out[i] = rg.cand_lo + i;
        if (tout) tout[i] = trow[rg.cand_lo + i];
      }
    } else if (!(n_sc * kChunkTop <= 1024
                     ? topk_summary_reg<256, 4>(uval + urow, uid + urow, uphys + urow, n_sc, rg.cand_lo,
                                                cand_hi, k, S, out, tout, tout != nullptr)
                     : topk_summary_reg<256, 8>(uval + urow, uid + urow, uphys + urow, n_sc, rg.cand_lo,
                                                cand_hi, k, S, out, tout, tout != nullptr))) {
      __syncthreads();
      topk_select<256, true>(scores + row * A.max_blocks + rg.cand_lo, n, k, rg.cand_lo, S, out, trow, tout);
    }
    if (threadIdx.x == 0) sel_count[row] = k;
    for (int i = k + (int)threadIdx.x; i < P.topk; i += 256) {
      out[i] = -1;
      if (tout) tout[i] = -1;
    }
  } else {
    topk_group<256, kStepTopkKeys, true>(P, scores, A.seq_lens, A.max_blocks, sel, sel_count, A.table,
                                         tiles, seq, grp, *reinterpret_cast<TopkLds*>(smem));
  }
  if (threadIdx.x == 0) st_coh(cp, 0);  // stored last: the selection's barriers would wait for it
  KVS_TL_MARK(3)
}

template <int G, int METHOD, int KV>
static void launch_ss_mq(const AttnArgs& A, dim3 grid, hipStream_t s, const void* reps, float* scores,
                         int32_t* sel, int32_t* cnt, int32_t* tiles, int* ctr, int ctr_stride, int n_sc, int n_il_wg,
                         int il_per, const Summaries& U) {
  if (U.val)  // SEPARATE long rows (checked by the caller)
    hipLaunchKernelGGL((score_select_kernel<G, METHOD, kSeparate, KV, true>), grid, dim3(256), 0, s, A, reps,
                       scores, sel, cnt, tiles, ctr, ctr_stride, n_sc, n_il_wg, il_per, U.val, U.id, U.phys);
  else if (A.P.mode == kSeparate)
    hipLaunchKernelGGL((score_select_kernel<G, METHOD, kSeparate, KV>), grid, dim3(256), 0, s, A, reps,
                       scores, sel, cnt, tiles, ctr, ctr_stride, n_sc, n_il_wg, il_per, U.val, U.id, U.phys);
  else
    hipLaunchKernelGGL((score_select_kernel<G, METHOD, kShared, KV>), grid, dim3(256), 0, s, A, reps,
                       scores, sel, cnt, tiles, ctr, ctr_stride, n_sc, n_il_wg, il_per, U.val, U.id, U.phys);
}

template <int G, int KV>
static void launch_ss_g(const AttnArgs& A, dim3 grid, hipStream_t s, const void* reps, float* scores,
                        int32_t* sel, int32_t* cnt, int32_t* tiles, int* ctr, int ctr_stride, int n_sc, int n_il_wg,
                        int il_per, const Summaries& U) {
  switch (A.P.method) {
    case kQuest: launch_ss_mq<G, kQuest, KV>(A, grid, s, reps, scores, sel, cnt, tiles, ctr, ctr_stride, n_sc, n_il_wg, il_per, U); break;
    case kMax: launch_ss_mq<G, kMax, KV>(A, grid, s, reps, scores, sel, cnt, tiles, ctr, ctr_stride, n_sc, n_il_wg, il_per, U); break;
    case kMean: launch_ss_mq<G, kMean, KV>(A, grid, s, reps, scores, sel, cnt, tiles, ctr, ctr_stride, n_sc, n_il_wg, il_per, U); break;
    default: launch_ss_mq<G, kFix, KV>(A, grid, s, reps, scores, sel, cnt, tiles, ctr, ctr_stride, n_sc, n_il_wg, il_per, U); break;
  }
}

template <int KV>
hipError_t launch_score_select_kv(const AttnArgs& A_in, const void* rep_pool, float* scores, int32_t* sel,
                                  int32_t* cnt, int32_t* tiles, int* ctr, int batch, hipStream_t s,
                                  const Summaries& U, int il_per) {
  AttnArgs A = A_in;
  A.P.tl_kind = kTlIlStep;
  const Params& P = A.P;
  const int sb = P.mode == kSeparate ? kScoreBlocksPerHeadWg : score_blocks_per_wg(P);
  const int n_sc = (A.max_blocks + sb - 1) / sb;
  if (il_per < 0 || il_per > A.n_il_max) il_per = A.n_il_max;
  const int n_il_wg = batch * P.Hkv * il_per;
  const dim3 grid(n_il_wg + batch * P.G * n_sc);
  const int cst = step_ctr_stride(batch * P.G);
  switch (P.g) {
    case 1: launch_ss_g<1, KV>(A, grid, s, rep_pool, scores, sel, cnt, tiles, ctr, cst, n_sc, n_il_wg, il_per, U); break;
    case 2: launch_ss_g<2, KV>(A, grid, s, rep_pool, scores, sel, cnt, tiles, ctr, cst, n_sc, n_il_wg, il_per, U); break;
    case 4: launch_ss_g<4, KV>(A, grid, s, rep_pool, scores, sel, cnt, tiles, ctr, cst, n_sc, n_il_wg, il_per, U); break;
    case 8: launch_ss_g<8, KV>(A, grid, s, rep_pool, scores, sel, cnt, tiles, ctr, cst, n_sc, n_il_wg, il_per, U); break;
    default: launch_ss_g<16, KV>(A, grid, s, rep_pool, scores, sel, cnt, tiles, ctr, cst, n_sc, n_il_wg, il_per, U); break;
  }
  return hipGetLastError();
}

// The selected tiles of a step whose score rows an earlier launch stored, and the Initial/Local tiles
// [il0, n_il_max) of every KV head, in one grid: workgroups [0, n_sel) are the selected tiles, entry i
// of the selection of KV head h of sequence seq at (seq * Hkv + h) * topk + i -- dispatched first, so
// their loads are not queued behind the Initial/Local tiles' stream -- then Initial/Local tile
// il0 + t at n_sel + (seq * Hkv + h) * (n_il_max - il0) + t.  A selected tile's workgroup makes its
// group's selection itself (every workgroup of a group makes the same one) and gathers its entry; the
// one of entry 0 (of KV head 0 for SHARED) also writes the group's selection and count.  Nothing
// passes between the workgroups of the launch.
//  * SRC kSrcRow (rows of up to kStepTopkSmall blocks): from the score row (topk_slot_reg);
//  * SRC kSrcSumm (SEPARATE rows up to kStepSummMax blocks): from the chunk summaries U of the scoring
//    launch (topk_summary_slot, n_u chunks per row), or, when a chunk holds more than kChunkTop of
//    the selection, from the whole score row (topk_select into LDS);
//  * SRC kSrcList (the confined step): from the preselected set of each row -- U.id = the sets
//    [rows][n_u] (block ids), U.val / U.phys = their scores and physical ids by position, stored by
//    the scoring launch (topk_list_slot).
constexpr int kSrcRow = 0, kSrcSumm = 1, kSrcList = 2;
template <int G, int KV, int KPT, int SRC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 4 : 2))) void attn_select_kernel(
    AttnArgs A, const float* __restrict__ scores, int32_t* __restrict__ sel, int32_t* __restrict__ sel_count,
    int n_sel, int il0, Summaries U, int n_u) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStepLds];
  __shared__ int s_slot[2];
  const Params& P = A.P;
  const int x = blockIdx.x;
  if (x >= n_sel) {
    const int il_n = A.n_il_max - il0, j = x - n_sel;
    attn_item<G, true, false, KV>(A, il0 + j % il_n, (j / il_n) % P.Hkv, j / (il_n * P.Hkv), smem, kTlAttnIl);
    return;
  }
  KVS_TL_BEGIN(P, kTlTileSel, 256)
  const int i = x % P.topk, h = (x / P.topk) % P.Hkv, seq = x / (P.topk * P.Hkv);
  const size_t row = (size_t)seq * P.G + (P.mode == kSeparate ? h : 0);
  const bool writer = i == 0 && (P.mode == kSeparate || h == 0);
  const int32_t* trow = A.table + (size_t)seq * A.max_blocks;
  TopkLds& S = *reinterpret_cast<TopkLds*>(smem);
  int2 e;
  if constexpr (SRC == kSrcList) {
    const Regions rg = regions_of(A.seq_lens[seq], P.initial_len, P.local_len);
    const size_t urow = row * n_u;
    e = topk_list_slot<256, KPT>(U.val + urow, U.phys + urow, U.id + urow, n_u, rg.cand_lo,
                                 min(rg.cand_hi, A.max_blocks), P.topk, i, S, s_slot, writer,
                                 sel + row * P.topk, sel_count + row);
  } else if constexpr (SRC == kSrcSumm) {
    const Regions rg = regions_of(A.seq_lens[seq], P.initial_len, P.local_len);
    const int lo = rg.cand_lo, hi = min(rg.cand_hi, A.max_blocks);
    const int n = max(0, hi - lo), k = min(P.topk, n);
    int32_t* srow = sel + row * P.topk;
    if (writer) {
      if (threadIdx.x == 0) sel_count[row] = k;
      for (int j = k + (int)threadIdx.x; j < P.topk; j += 256) srow[j] = -1;
    }
    if (i >= k) return;
    if (k >= n) {  // every candidate
      if (writer)
        for (int j = threadIdx.x; j < n; j += 256) srow[j] = lo + j;
      e = make_int2(lo + i, trow[lo + i]);
    } else {
      const size_t urow = row * n_u * kChunkTop;
      if (topk_summary_slot<256, KPT>(U.val + urow, U.id + urow, U.phys + urow, n_u, lo, hi, k, i, S, s_slot,
                                      writer, srow)) {
        e = make_int2(s_slot[0], s_slot[1]);
      } else {  // a chunk overflows: the whole row, its selection and physical ids into LDS after S
        int32_t* lsel = reinterpret_cast<int32_t*>(smem + kSummSlotOff);
        int32_t* ltile = lsel + P.topk;
        __syncthreads();
        topk_select<256>(scores + row * A.max_blocks + lo, n, k, lo, S, lsel, trow, ltile);
        __syncthreads();
        e = make_int2(lsel[i], ltile[i]);
        if (writer)
          for (int j = threadIdx.x; j < k; j += 256) srow[j] = lsel[j];
      }
    }
  } else {
    e = topk_slot_reg<256, KPT>(scores + row * A.max_blocks, A.max_blocks, A.seq_lens + seq, P.initial_len,
                                P.local_len, P.topk, i, S, trow, writer, sel + row * P.topk, sel_count + row,
                                s_slot, KVS_TL_REC);
  }
  KVS_TL_MARK(3)
  if (e.x < 0) return;
  const TileList tl = tiles_of(A.seq_lens[seq], P, 0);
  const int part = tl.nI + tl.nLoc + i;
  const size_t head0 = (size_t)seq * P.Hq + (size_t)h * G;
  float* po = A.part_o + head0 * A.max_parts * kDim;
  float* pml = A.part_ml + head0 * A.max_parts * 2;
  if (e.y < 0) {  // a table entry that names no block
    empty_partial<G>(po, pml, A.max_parts, part);
    return;
  }
  __syncthreads();  // the selection's LDS becomes the tile's
  attn_tile<G, KV>(P, A.q + head0 * kDim, A.k_pool, A.v_pool, h, e.y, kBlock, po, pml, A.max_parts, part, smem);
}

template <int KV>
hipError_t launch_attn_select_kv(const AttnArgs& A_in, const float* scores, int32_t* sel, int32_t* sel_count,
                                 int batch, int il0, hipStream_t s, const Summaries& U, int n_list) {
  AttnArgs A = A_in;
  A.P.tl_kind = kTlAttn;
  if (il0 < 0 || il0 > A.n_il_max) il0 = A.n_il_max;
  const int n_sel = batch * A.P.Hkv * A.P.topk;
  const dim3 grid(n_sel + batch * A.P.Hkv * (A.n_il_max - il0));
  if (n_list > 0) {  // preselected sets of up to 256 (KPT 1) or 1024 (KPT 4) entries
#define KVS_ASL(GG, KK)                                                                              \
  hipLaunchKernelGGL((attn_select_kernel<GG, KV, KK, kSrcList>), grid, dim3(256), 0, s, A, scores, sel, \
                     sel_count, n_sel, il0, U, n_list)
#define KVS_ASL_G(GG)                    \
  if (n_list <= 256) KVS_ASL(GG, 1);     \
  else KVS_ASL(GG, 4);
    switch (A.P.g) {
      case 1: KVS_ASL_G(1); break;
      case 2: KVS_ASL_G(2); break;
      case 4: KVS_ASL_G(4); break;
      case 8: KVS_ASL_G(8); break;
      default: KVS_ASL_G(16); break;
    }
#undef KVS_ASL_G
#undef KVS_ASL
    return hipGetLastError();
  }
  const int n_sc = (A.max_blocks + kChunkBlocks - 1) / kChunkBlocks;
  if (U.val) {  // summaries of up to 256 * 4 (KPT 4) or 256 * 8 entries per row
    const int kpt = n_sc * kChunkTop <= 1024 ? 4 : 8;
#define KVS_ASU(GG, KK)                                                                              \
  hipLaunchKernelGGL((attn_select_kernel<GG, KV, KK, kSrcSumm>), grid, dim3(256), 0, s, A, scores, sel, \
                     sel_count, n_sel, il0, U, n_sc)
#define KVS_ASU_G(GG)                    \
  if (kpt == 4) KVS_ASU(GG, 4);          \
  else KVS_ASU(GG, 8);
    switch (A.P.g) {
      case 1: KVS_ASU_G(1); break;
      case 2: KVS_ASU_G(2); break;
      case 4: KVS_ASU_G(4); break;
      case 8: KVS_ASU_G(8); break;
      default: KVS_ASU_G(16); break;
    }
#undef KVS_ASU_G
#undef KVS_ASU
    return hipGetLastError();
  }
  const int kpt = A.max_blocks <= 256 ? 1 : (A.max_blocks <= 1024 ? 4 : 8);
#define KVS_AS(GG, KK)                                                                             \
  hipLaunchKernelGGL((attn_select_kernel<GG, KV, KK, kSrcRow>), grid, dim3(256), 0, s, A, scores, sel, \
                     sel_count, n_sel, il0, U, n_sc)
#define KVS_AS_G(GG)                       \
  if (kpt == 1) KVS_AS(GG, 1);             \
  else if (kpt == 4) KVS_AS(GG, 4);        \
  else KVS_AS(GG, 8);
  switch (A.P.g) {
    case 1: KVS_AS_G(1); break;
    case 2: KVS_AS_G(2); break;
    case 4: KVS_AS_G(4); break;
    case 8: KVS_AS_G(8); break;
    default: KVS_AS_G(16); break;
  }
#undef KVS_AS_G
#undef KVS_AS
  return hipGetLastError();
}

// Long rows: the selections, in 512-lane workgroups, and the Initial/Local tiles in one grid.
// Workgroups [0, n_topk) are the (sequence, group) selections (keys in registers up to 16 per lane);
// each later workgroup runs two Initial/Local tiles, one per 256-lane half, from the flat index
// (seq * Hkv + h) * n_il_max + t.  A half without a tile (past the sequence's own count or the end)
// still takes part in the barriers: it computes an empty tile and stores nothing.  Two halves (73 KiB
// of LDS) rather than four quarters per workgroup let the tiles spread over twice as many CUs.
template <int G, int KV>
__global__ __launch_bounds__(512) void topk_il_wide_kernel(AttnArgs A, const float* __restrict__ scores,
                                                            int32_t* __restrict__ sel,
                                                            int32_t* __restrict__ sel_count,
                                                            int32_t* __restrict__ tiles, int n_topk,
                                                            int n_il_total) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kAttnLdsBytes];
  const Params& P = A.P;
  const int x = blockIdx.x;
  if (x < n_topk) {
    KVS_TL_BEGIN(P, kTlWideTopk, 512)
    topk_group<512, 16>(P, scores, A.seq_lens, A.max_blocks, sel, sel_count, A.table, tiles, x / P.G,
                         x % P.G, *reinterpret_cast<TopkLds*>(smem));
    KVS_TL_MARK(3)
    return;
  }
  const int f = (x - n_topk) * 2 + (threadIdx.x >> 8);  // this half's flat tile index
  const bool in = f < n_il_total;
  const int fi = in ? f : 0;
  const int seq = fi / (P.Hkv * A.n_il_max), h = (fi / A.n_il_max) % P.Hkv, t = fi % A.n_il_max;
  const TileList tl = tiles_of(A.seq_lens[seq], P, 0);
  const bool have = in && t < tl.nI + tl.nLoc;
  int phys = 0, ntok = 0;
  if (have) {
    const int2 lt = il_tile(tl, t);
    const int v = lt.x < A.max_blocks ? A.table[(size_t)seq * A.max_blocks + lt.x] : -1;
    phys = v < 0 ? 0 : v;   // an invalid table entry gives an empty partial
    ntok = v < 0 ? 0 : lt.y;
  }
  const size_t head0 = (size_t)seq * P.Hq + (size_t)h * G;
  attn_tile<G, KV>(P, A.q + head0 * kDim, A.k_pool, A.v_pool, h, phys, ntok,
               A.part_o + head0 * A.max_parts * kDim, A.part_ml + head0 * A.max_parts * 2, A.max_parts,
               t, smem + (threadIdx.x >> 8) * kAttnLdsBytes, have);
}

template <int KV>
hipError_t launch_topk_il_wide_kv(const AttnArgs& A_in, const float* scores, int32_t* sel, int32_t* sel_count,
                                  int32_t* tiles, int batch, hipStream_t s) {
  AttnArgs A = A_in;
  A.P.tl_kind = kTlIlWide;
  const int n_topk = A.P.G * batch;
  const int n_il_total = batch * A.P.Hkv * A.n_il_max;
  const dim3 grid(n_topk + (n_il_total + 1) / 2), block(512);
#define KVS_WIDE(GG)                                                                                 \
  hipLaunchKernelGGL((topk_il_wide_kernel<GG, KV>), grid, block, 0, s, A, scores, sel, sel_count, tiles, \
                     n_topk, n_il_total)
  switch (A.P.g) {
    case 1: KVS_WIDE(1); break;
    case 2: KVS_WIDE(2); break;
    case 4: KVS_WIDE(4); break;
    case 8: KVS_WIDE(8); break;
    default: KVS_WIDE(16); break;
  }
#undef KVS_WIDE
  return hipGetLastError();
}

// The first launch of the confined decode step (kvs_decode_step_preselected) for sets of up to
// kPreselStepMax entries: n_pc scoring workgroups per (sequence, group) row score the row's
// preselected blocks -- positions [c * sb, c * sb + sb) of presel[row] -- and store each score and
// physical id by position, coherently (cs, cph [row][n_presel]); the one that brings the row's
// counter to n_pc selects from them (topk_list_reg) and resets it.  With sel null the kernel only
// scores (the selections are made by the tiles' workgroups).  Then the Initial/Local tiles [0, il_per)
// of each KV head, as in score_select_kernel.  Rows of any length: only the set is scored.
template <int G, int METHOD, int MODE, int KV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 4 : 2))) void presel_step_kernel(
    AttnArgs A, const void* __restrict__ rep_pool, const int32_t* __restrict__ presel, int n_presel,
    float* __restrict__ cs, int32_t* __restrict__ cph, int32_t* __restrict__ sel,
    int32_t* __restrict__ sel_count, int32_t* __restrict__ tiles, int* __restrict__ ctr, int ctr_stride,
    int n_pc, int n_il_wg, int il_per) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStepLds];
  __shared__ int s_last;
  const Params& P = A.P;
  const int n_score_wg = (int)gridDim.x - n_il_wg;
  const int x = blockIdx.x;
  if (x >= n_score_wg) {
    const int xi = x - n_score_wg;
    const int per_seq = P.Hkv * il_per;
    const int r = xi % per_seq;
    attn_item<G, true, false, KV>(A, r % il_per, r / il_per, xi / per_seq, smem);
    return;
  }
  constexpr bool SEP = MODE == kSeparate;
  KVS_TL_BEGIN(P, kTlScoreSel, 256)
  const int row = x / n_pc, c = x % n_pc;
  const int seq = row / P.G, grp = row % P.G;
  const int sb = SEP ? kScoreBlocksPerHeadWg : score_blocks_per_wg(P);
  const int32_t* trow = A.table + (size_t)seq * A.max_blocks;
  const int32_t* ids = presel + (size_t)row * n_presel;
  const size_t rbase = (size_t)seq * P.G * n_presel;  // score rows of the sequence's groups
  score_blocks_range<G, METHOD, MODE, SEP, true, true>(P, A.q + (size_t)seq * P.Hq * kDim, rep_pool, trow,
                                                       A.max_blocks, A.seq_lens[seq], c * sb, sb, cs + rbase,
                                                       reinterpret_cast<float*>(smem), grp, nullptr, ids,
                                                       n_presel, cph + rbase);
  KVS_TL_MARK_LOADED(1)
  if (sel == nullptr) return;  // scores only: the selections are made by the tiles' workgroups
  wait_mem();
  __syncthreads();
  int* cp = ctr + (size_t)row * ctr_stride;
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(cp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n_pc - 1;
  __syncthreads();
  KVS_TL_MARK(2)
  if (!s_last) return;  // else every scoring workgroup of the row has arrived
  const Regions rg = regions_of(A.seq_lens[seq], P.initial_len, P.local_len);
  topk_list_reg<256, kPreselStepKeys>(cs + (size_t)row * n_presel, cph + (size_t)row * n_presel, ids,
                                      n_presel, rg.cand_lo, min(rg.cand_hi, A.max_blocks), P.topk,
                                      *reinterpret_cast<TopkLds*>(smem), sel + (size_t)row * P.topk,
                                      sel_count + row, tiles + (size_t)row * P.topk);
  if (threadIdx.x == 0) st_coh(cp, 0);  // stored last: the selection's barriers would wait for it
  KVS_TL_MARK(3)
}

template <int KV>
hipError_t launch_presel_step_kv(const AttnArgs& A_in, const void* rep_pool, const int32_t* presel,
                                 int n_presel, float* cs, int32_t* cph, int32_t* sel, int32_t* cnt,
                                 int32_t* tiles, int* ctr, int batch, hipStream_t s, int il_per) {
  AttnArgs A = A_in;
  A.P.tl_kind = kTlIlStep;
  const Params& P = A.P;
  const int sb = P.mode == kSeparate ? kScoreBlocksPerHeadWg : score_blocks_per_wg(P);
  const int n_pc = (n_presel + sb - 1) / sb;
  const int rows = batch * P.G;
  if (il_per < 0 || il_per > A.n_il_max) il_per = A.n_il_max;
  const int n_il_wg = batch * P.Hkv * il_per;
  const dim3 grid(n_il_wg + rows * n_pc);
  const int cst = step_ctr_stride(rows);
#define KVS_PS(GG, MM, MO)                                                                            \
  hipLaunchKernelGGL((presel_step_kernel<GG, MM, MO, KV>), grid, dim3(256), 0, s, A, rep_pool, presel, \
                     n_presel, cs, cph, sel, cnt, tiles, ctr, cst, n_pc, n_il_wg, il_per)
#define KVS_PS_M(GG, MO)                               \
  switch (P.method) {                                  \
    case kQuest: KVS_PS(GG, kQuest, MO); break;        \
    case kMax: KVS_PS(GG, kMax, MO); break;            \
    case kMean: KVS_PS(GG, kMean, MO); break;          \
    default: KVS_PS(GG, kFix, MO); break;              \
  }
#define KVS_PS_G(GG)                                                          \
  if (P.mode == kSeparate) { KVS_PS_M(GG, kSeparate) } else { KVS_PS_M(GG, kShared) }
  switch (P.g) {
    case 1: KVS_PS_G(1); break;
    case 2: KVS_PS_G(2); break;
    case 4: KVS_PS_G(4); break;
    case 8: KVS_PS_G(8); break;
    default: KVS_PS_G(16); break;
  }
#undef KVS_PS_G
#undef KVS_PS_M
#undef KVS_PS
  return hipGetLastError();
}

}  // namespace kvs
