// kvs_decode_step, first launch: block scoring and the Initial/Local attention tiles in one grid.
// The two need nothing from each other -- Initial and Local are attended whatever the selection
// [KT-LC §4.2] -- so the gather of Initial/Local K/V overlaps the scoring.  Workgroups
// [0, n_score) of sequence seq score sb blocks each (score_core.h); the rest are Initial/Local tiles
// (attn_core.h), the x-th tile of KV head h at x + h * n_il_max.  The step then runs top-k (which
// also writes the selected tiles' physical ids), the selected tiles and the merge.
#include "attn_core.h"
#include "kvs_launch.h"
#include "score_core.h"

namespace kvs {

// 4 workgroups per CU (the attention tiles' occupancy) unless the scoring of 8 or 16 query heads per
// KV head needs more registers.
template <int G, int METHOD, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 4 : 2))) void score_il_kernel(AttnArgs A, const void* __restrict__ rep_pool,
                                                       float* __restrict__ scores, int sb, int n_score) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kAttnLdsBytes];
  const int seq = blockIdx.y;
  const int x = blockIdx.x;
  if (x < n_score) {
    const Params& P = A.P;
    score_blocks_range<G, METHOD, MODE>(P, A.q + (size_t)seq * P.Hq * kDim, rep_pool,
                                        A.table + (size_t)seq * A.max_blocks, A.max_blocks,
                                        A.seq_lens[seq], x * sb, sb,
                                        scores + (size_t)seq * P.G * A.max_blocks,
                                        reinterpret_cast<float*>(smem));
  } else {
    const int y = x - n_score;
    attn_item<G, true, false>(A, y % A.n_il_max, y / A.n_il_max, seq, smem);
  }
}

template <int G, int METHOD>
static void launch_si_m(const AttnArgs& A, dim3 grid, hipStream_t s, const void* reps, float* scores,
                        int sb, int n_score) {
  if (A.P.mode == kSeparate)
    hipLaunchKernelGGL((score_il_kernel<G, METHOD, kSeparate>), grid, dim3(256), 0, s, A, reps, scores, sb, n_score);
  else
    hipLaunchKernelGGL((score_il_kernel<G, METHOD, kShared>), grid, dim3(256), 0, s, A, reps, scores, sb, n_score);
}

template <int G>
static void launch_si_g(const AttnArgs& A, dim3 grid, hipStream_t s, const void* reps, float* scores,
                        int sb, int n_score) {
  switch (A.P.method) {
    case kQuest: launch_si_m<G, kQuest>(A, grid, s, reps, scores, sb, n_score); break;
    case kMax: launch_si_m<G, kMax>(A, grid, s, reps, scores, sb, n_score); break;
    case kMean: launch_si_m<G, kMean>(A, grid, s, reps, scores, sb, n_score); break;
    default: launch_si_m<G, kFix>(A, grid, s, reps, scores, sb, n_score); break;
  }
}

hipError_t launch_score_il(const AttnArgs& A, const void* rep_pool, float* scores, int batch,
                           hipStream_t s) {
  const int sb = score_blocks_per_wg(A.P);
  const int n_score = (A.max_blocks + sb - 1) / sb;
  const dim3 grid(n_score + A.P.Hkv * A.n_il_max, batch);
  switch (A.P.g) {
    case 1: launch_si_g<1>(A, grid, s, rep_pool, scores, sb, n_score); break;
    case 2: launch_si_g<2>(A, grid, s, rep_pool, scores, sb, n_score); break;
    case 4: launch_si_g<4>(A, grid, s, rep_pool, scores, sb, n_score); break;
    case 8: launch_si_g<8>(A, grid, s, rep_pool, scores, sb, n_score); break;
    default: launch_si_g<16>(A, grid, s, rep_pool, scores, sb, n_score); break;
  }
  return hipGetLastError();
}

}  // namespace kvs
