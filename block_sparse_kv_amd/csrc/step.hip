// kvs_decode_step: scoring -> top-k -> attention tiles -> merge, with the Initial/Local tiles -- which
// do not depend on the selection [KT-LC §4.2] -- placed where their K/V gather costs least:
//  * short rows (max_blocks <= kStepTopkSmall): in the top-k launch (topk_il_kernel).  Their gather
//    then runs while the few top-k workgroups -- one per (sequence, group), 256 lanes, keys in
//    registers -- choose the blocks;
//  * long rows: in the selected-tile launch, whose stream they lengthen by their bytes only, while
//    top-k gets 1024-lane workgroups (topk.hip).
// In every grid an attention tile is one workgroup (attn_core.h).
#include "attn_core.h"
#include "kvs_launch.h"
#include "topk_core.h"

namespace kvs {

constexpr int kStepTopkKeys = 8;  // keys per lane of the 256-lane selections
constexpr int kStepTopkSmall = 256 * kStepTopkKeys;
constexpr int kStepLds = kAttnLdsBytes > (int)sizeof(TopkLds) ? kAttnLdsBytes : (int)sizeof(TopkLds);

template <int G>
__global__ __launch_bounds__(256) void topk_il_kernel(AttnArgs A, const float* __restrict__ scores,
                                                      int32_t* __restrict__ sel,
                                                      int32_t* __restrict__ sel_count,
                                                      int32_t* __restrict__ tiles, int n_topk) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStepLds];
  const Params& P = A.P;
  const int x = blockIdx.x;
  if (x < n_topk) {
    topk_group<256, kStepTopkKeys>(P, scores, A.seq_lens, A.max_blocks, sel, sel_count, A.table, tiles,
                                   x / P.G, x % P.G, *reinterpret_cast<TopkLds*>(smem));
  } else {
    const int y = x - n_topk;
    const int per_seq = P.Hkv * A.n_il_max;
    const int r = y % per_seq;
    attn_item<G, true, false>(A, r % A.n_il_max, r / A.n_il_max, y / per_seq, smem);
  }
}

hipError_t launch_topk_il(const AttnArgs& A, const float* scores, int32_t* sel, int32_t* sel_count,
                          int32_t* tiles, int batch, hipStream_t s) {
  const int n_topk = A.P.G * batch;
  const dim3 grid(n_topk + batch * A.P.Hkv * A.n_il_max), block(256);
  switch (A.P.g) {
    case 1: hipLaunchKernelGGL(topk_il_kernel<1>, grid, block, 0, s, A, scores, sel, sel_count, tiles, n_topk); break;
    case 2: hipLaunchKernelGGL(topk_il_kernel<2>, grid, block, 0, s, A, scores, sel, sel_count, tiles, n_topk); break;
    case 4: hipLaunchKernelGGL(topk_il_kernel<4>, grid, block, 0, s, A, scores, sel, sel_count, tiles, n_topk); break;
    case 8: hipLaunchKernelGGL(topk_il_kernel<8>, grid, block, 0, s, A, scores, sel, sel_count, tiles, n_topk); break;
    default: hipLaunchKernelGGL(topk_il_kernel<16>, grid, block, 0, s, A, scores, sel, sel_count, tiles, n_topk); break;
  }
  return hipGetLastError();
}


hipError_t launch_decode_step(const AttnArgs& A, const void* rep_pool, float* scores, int32_t* sel,
                              int32_t* sel_count, int32_t* tiles, int batch, hipStream_t s) {
  const Params& P = A.P;
  int32_t* tl = P.topk > 0 ? tiles : nullptr;
  hipError_t e = launch_score(P, A.q, rep_pool, A.table, A.max_blocks, A.seq_lens, batch, scores, s);
  if (A.max_blocks <= kStepTopkSmall) {
    if (e == hipSuccess) e = launch_topk_il(A, scores, sel, sel_count, tl, batch, s);
    if (e == hipSuccess) e = launch_attn_tiles(A, batch, false, true, s);
  } else {
    if (e == hipSuccess)
      e = launch_topk(P, scores, A.seq_lens, batch, A.max_blocks, sel, sel_count, A.table, tl, s);
    if (e == hipSuccess) e = launch_attn_tiles(A, batch, true, true, s);
  }
  if (e == hipSuccess) e = launch_merge(A, batch, s);
  return e;
}

}  // namespace kvs
