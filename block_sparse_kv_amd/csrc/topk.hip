// Top-k kernel of kvs_topk_blocks and kvs_decode_step: one workgroup of 1024 lanes per (sequence,
// selection group); the selection itself is topk_group (topk_core.h).  With a table, the physical ids
// of the selected blocks are written too (for the attention that follows in kvs_decode_step).
#include "kvs_launch.h"
#include "topk_core.h"

namespace kvs {

constexpr int kTopkThreads = 1024;  // up to 16 candidates per lane stay in registers; more are re-read

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(Params P, const float* __restrict__ scores,
                                                            const int32_t* __restrict__ seq_lens,
                                                            int max_blocks, int32_t* __restrict__ sel,
                                                            int32_t* __restrict__ sel_count,
                                                            const int32_t* __restrict__ table,
                                                            int32_t* __restrict__ tiles) {
  __shared__ TopkLds S;
  topk_group<kTopkThreads, 16>(P, scores, seq_lens, max_blocks, sel, sel_count, table, tiles,
                               blockIdx.y, blockIdx.x, S);
}

hipError_t launch_topk(const Params& P, const float* scores, const int32_t* seq_lens, int batch,
                       int max_blocks, int32_t* sel, int32_t* sel_count, const int32_t* table,
                       int32_t* tiles, hipStream_t s) {
  const dim3 grid(P.G, batch), block(kTopkThreads);
  hipLaunchKernelGGL(topk_kernel, grid, block, 0, s, P, scores, seq_lens, max_blocks, sel, sel_count,
                     table, tiles);
  return hipGetLastError();
}

}  // namespace kvs
