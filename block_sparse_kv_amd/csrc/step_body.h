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

// First the scoring workgroups, n_sc per (sequence, group), over every KV head (SHARED) or over one KV
// head (SEPARATE; group = KV head): dispatched first, their few loads are not queued behind the
// tiles' stream.  With sel null the kernel only scores and streams the tiles (a selection made by
// later launches).  Then n_il_wg Initial/Local tiles, tile t of KV head h of sequence seq at
// (seq * Hkv + h) * n_il_max + t.  A scoring workgroup stores its
// scores coherently, waits for them to complete and bumps the group's counter; the one that brings it
// to n_sc resets it and selects.  Nothing waits on another workgroup.
template <int G, int METHOD, int MODE, int KV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 4 : 2))) void score_select_kernel(
    AttnArgs A, const void* __restrict__ rep_pool, float* __restrict__ scores, int32_t* __restrict__ sel,
    int32_t* __restrict__ sel_count, int32_t* __restrict__ tiles, int* __restrict__ ctr, int n_sc,
    int n_il_wg) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStepLds];
  __shared__ int s_last;
  const Params& P = A.P;
  const int n_score_wg = (int)gridDim.x - n_il_wg;
  const int x = blockIdx.x;
  if (x >= n_score_wg) {
    const int xi = x - n_score_wg;
    const int per_seq = P.Hkv * A.n_il_max;
    const int r = xi % per_seq;
    attn_item<G, true, false, KV>(A, r % A.n_il_max, r / A.n_il_max, xi / per_seq, smem);
    return;
  }
  constexpr bool SEP = MODE == kSeparate;
  const int y = x;
  const int per_seq = P.G * n_sc;
  const int seq = y / per_seq, grp = (y % per_seq) / n_sc, c = y % n_sc;
  const int sb = SEP ? kScoreBlocksPerHeadWg : score_blocks_per_wg(P);
  score_blocks_range<G, METHOD, MODE, SEP, true>(P, A.q + (size_t)seq * P.Hq * kDim, rep_pool,
                                                 A.table + (size_t)seq * A.max_blocks, A.max_blocks,
                                                 A.seq_lens[seq], c * sb, sb,
                                                 scores + (size_t)seq * P.G * A.max_blocks,
                                                 reinterpret_cast<float*>(smem), grp);
  if (sel == nullptr) return;  // scores and Initial/Local tiles only: the selection comes later
  wait_mem();
  __syncthreads();
  int* cp = ctr + (size_t)seq * P.G + grp;
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(cp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n_sc - 1;
  __syncthreads();
  if (!s_last) return;  // else every scoring workgroup of the group has arrived
  topk_group<256, kStepTopkKeys, true>(P, scores, A.seq_lens, A.max_blocks, sel, sel_count, A.table,
                                       tiles, seq, grp, *reinterpret_cast<TopkLds*>(smem));
  if (threadIdx.x == 0) st_coh(cp, 0);  // stored last: the selection's barriers would wait for it
}

template <int G, int METHOD, int KV>
static void launch_ss_mq(const AttnArgs& A, dim3 grid, hipStream_t s, const void* reps, float* scores,
                         int32_t* sel, int32_t* cnt, int32_t* tiles, int* ctr, int n_sc, int n_il_wg) {
  if (A.P.mode == kSeparate)
    hipLaunchKernelGGL((score_select_kernel<G, METHOD, kSeparate, KV>), grid, dim3(256), 0, s, A, reps,
                       scores, sel, cnt, tiles, ctr, n_sc, n_il_wg);
  else
    hipLaunchKernelGGL((score_select_kernel<G, METHOD, kShared, KV>), grid, dim3(256), 0, s, A, reps,
                       scores, sel, cnt, tiles, ctr, n_sc, n_il_wg);
}

template <int G, int KV>
static void launch_ss_g(const AttnArgs& A, dim3 grid, hipStream_t s, const void* reps, float* scores,
                        int32_t* sel, int32_t* cnt, int32_t* tiles, int* ctr, int n_sc, int n_il_wg) {
  switch (A.P.method) {
    case kQuest: launch_ss_mq<G, kQuest, KV>(A, grid, s, reps, scores, sel, cnt, tiles, ctr, n_sc, n_il_wg); break;
    case kMax: launch_ss_mq<G, kMax, KV>(A, grid, s, reps, scores, sel, cnt, tiles, ctr, n_sc, n_il_wg); break;
    case kMean: launch_ss_mq<G, kMean, KV>(A, grid, s, reps, scores, sel, cnt, tiles, ctr, n_sc, n_il_wg); break;
    default: launch_ss_mq<G, kFix, KV>(A, grid, s, reps, scores, sel, cnt, tiles, ctr, n_sc, n_il_wg); break;
  }
}

template <int KV>
hipError_t launch_score_select_kv(const AttnArgs& A, const void* rep_pool, float* scores, int32_t* sel,
                                  int32_t* cnt, int32_t* tiles, int* ctr, int batch, hipStream_t s) {
  const Params& P = A.P;
  const int sb = P.mode == kSeparate ? kScoreBlocksPerHeadWg : score_blocks_per_wg(P);
  const int n_sc = (A.max_blocks + sb - 1) / sb;
  const int n_il_wg = batch * P.Hkv * A.n_il_max;
  const dim3 grid(n_il_wg + batch * P.G * n_sc);
  switch (P.g) {
    case 1: launch_ss_g<1, KV>(A, grid, s, rep_pool, scores, sel, cnt, tiles, ctr, n_sc, n_il_wg); break;
    case 2: launch_ss_g<2, KV>(A, grid, s, rep_pool, scores, sel, cnt, tiles, ctr, n_sc, n_il_wg); break;
    case 4: launch_ss_g<4, KV>(A, grid, s, rep_pool, scores, sel, cnt, tiles, ctr, n_sc, n_il_wg); break;
    case 8: launch_ss_g<8, KV>(A, grid, s, rep_pool, scores, sel, cnt, tiles, ctr, n_sc, n_il_wg); break;
    default: launch_ss_g<16, KV>(A, grid, s, rep_pool, scores, sel, cnt, tiles, ctr, n_sc, n_il_wg); break;
  }
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
    topk_group<512, 16>(P, scores, A.seq_lens, A.max_blocks, sel, sel_count, A.table, tiles, x / P.G,
                         x % P.G, *reinterpret_cast<TopkLds*>(smem));
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
hipError_t launch_topk_il_wide_kv(const AttnArgs& A, const float* scores, int32_t* sel, int32_t* sel_count,
                                  int32_t* tiles, int batch, hipStream_t s) {
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

}  // namespace kvs
