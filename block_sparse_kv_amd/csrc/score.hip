// kvs_score_blocks kernel: one workgroup per (chunk of score_blocks_per_wg blocks, sequence); the
// scoring itself is score_blocks_range (score_core.h).
#include "kvs_launch.h"
#include "score_core.h"

namespace kvs {

template <int G, int METHOD, int MODE>
__global__ __launch_bounds__(256) void score_kernel(Params P, const uint16_t* __restrict__ q,
                                                    const void* __restrict__ rep_pool,
                                                    const int32_t* __restrict__ table, int max_blocks,
                                                    const int32_t* __restrict__ seq_lens,
                                                    float* __restrict__ scores) {
  __shared__ float part[16 * kScorePasses];
  KVS_TL_BEGIN(P, kTlScore, 256)
  const int seq = blockIdx.y;
  const int sb = score_blocks_per_wg(P);
  score_blocks_range<G, METHOD, MODE>(P, q + (size_t)seq * P.Hq * kDim, rep_pool,
                                      table + (size_t)seq * max_blocks, max_blocks, seq_lens[seq],
                                      blockIdx.x * sb, sb, scores + (size_t)seq * P.G * max_blocks,
                                      part);
  KVS_TL_MARK_LOADED(1)
}

template <int G, int METHOD>
static void launch_score_m(const Params& P, dim3 grid, hipStream_t s, const uint16_t* q,
                           const void* reps, const int32_t* table, int mb, const int32_t* lens,
                           float* scores) {
  if (P.mode == kSeparate)
    hipLaunchKernelGGL((score_kernel<G, METHOD, kSeparate>), grid, dim3(256), 0, s, P, q, reps, table, mb, lens, scores);
  else
    hipLaunchKernelGGL((score_kernel<G, METHOD, kShared>), grid, dim3(256), 0, s, P, q, reps, table, mb, lens, scores);
}

template <int G>
static void launch_score_g(const Params& P, dim3 grid, hipStream_t s, const uint16_t* q,
                           const void* reps, const int32_t* table, int mb, const int32_t* lens,
                           float* scores) {
  switch (P.method) {
    case kQuest: launch_score_m<G, kQuest>(P, grid, s, q, reps, table, mb, lens, scores); break;
    case kMax: launch_score_m<G, kMax>(P, grid, s, q, reps, table, mb, lens, scores); break;
    case kMean: launch_score_m<G, kMean>(P, grid, s, q, reps, table, mb, lens, scores); break;
    default: launch_score_m<G, kFix>(P, grid, s, q, reps, table, mb, lens, scores); break;
  }
}

hipError_t launch_score(const Params& P, const void* q, const void* rep_pool,
                        const int32_t* table, int max_blocks, const int32_t* seq_lens, int batch,
                        float* scores, hipStream_t s) {
  const int sb = score_blocks_per_wg(P);
  const dim3 grid((max_blocks + sb - 1) / sb, batch);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  switch (P.g) {
    case 1: launch_score_g<1>(P, grid, s, qq, rep_pool, table, max_blocks, seq_lens, scores); break;
    case 2: launch_score_g<2>(P, grid, s, qq, rep_pool, table, max_blocks, seq_lens, scores); break;
    case 4: launch_score_g<4>(P, grid, s, qq, rep_pool, table, max_blocks, seq_lens, scores); break;
    case 8: launch_score_g<8>(P, grid, s, qq, rep_pool, table, max_blocks, seq_lens, scores); break;
    default: launch_score_g<16>(P, grid, s, qq, rep_pool, table, max_blocks, seq_lens, scores); break;
  }
  return hipGetLastError();
}

}  // namespace kvs
