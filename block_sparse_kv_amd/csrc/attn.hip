// Attention kernels over the per-tile work items of attn_core.h:
//  * attn_tiles_kernel: workgroup (x, h, seq) is one attended tile of KV head h -- the x-th
//    Initial/Local tile, or a selected one -- and writes one partial per query head of h;
//  * merge_wave_kernel: one wave per (query head, 16 channels) folds that slice of the head's
//    partials into out; merge_kernel, for partial counts whose weights do not fit the waves' LDS:
//    workgroup (j * 4 + q, seq) folds channels [32q, 32q + 32).
// kvs_sparse_decode_attn runs both (Initial/Local and selected tiles in one grid, selections as logical
// ids); kvs_decode_step runs them with the selections as physical ids, the Initial/Local tiles here
// or in its top-k launch (step.hip).
#include "attn_core.h"
#include "kvs_launch.h"

namespace kvs {

template <int G, bool IL, bool PHYS, int KV>
__global__ __launch_bounds__(256) void attn_tiles_kernel(AttnArgs A) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kAttnLdsBytes];
  attn_item<G, IL, PHYS, KV>(A, blockIdx.x, blockIdx.y, blockIdx.z, smem);
}

__global__ __launch_bounds__(256) void merge_kernel(AttnArgs A) {
  __shared__ __attribute__((aligned(16))) float lds[kMergeLdsFloats];
  constexpr int Q = kDim / kMergeCh;
  merge_item(A, blockIdx.x / Q, blockIdx.x % Q, blockIdx.y, lds);
}

// One wave per (query head, 16 channels), two per workgroup (spread over many CUs): wave w of
// workgroup x merges item 2x + w = (seq * Hq + j) * 8 + c.  Used when the waves' LDS (partial
// weights and the fold) fits.
constexpr int kMergeWaveLds = 65536;
__global__ __launch_bounds__(128) void merge_wave_kernel(AttnArgs A, int n_items) {
  extern __shared__ __attribute__((aligned(16))) float wlds[];
  const int item = blockIdx.x * 2 + (threadIdx.x >> 6);
  KVS_TL_BEGIN(A.P, kTlMerge, 128)
  if (item >= n_items) return;
  constexpr int C = kDim / kMergeChWave;
  const int c = item % C, j = (item / C) % A.P.Hq, seq = item / (C * A.P.Hq);
  merge_item_wave(A, j, c, seq, wlds + (threadIdx.x >> 6) * (A.max_parts + 256), KVS_TL_REC);
  KVS_TL_MARK(2)
}

AttnPlan attn_plan(const Params& P, int batch, int max_blocks) {
  const int nI = (P.initial_len + kBlock - 1) / kBlock;
  const int nLoc = (P.local_len + 2 * kBlock - 2) / kBlock;
  AttnPlan a;
  a.n_il_max = nI + nLoc < max_blocks ? nI + nLoc : max_blocks;
  a.max_parts = a.n_il_max + P.topk;
  a.part_o_bytes = (size_t)batch * P.Hq * a.max_parts * kDim * sizeof(float);
  a.part_ml_bytes = (size_t)batch * P.Hq * a.max_parts * 2 * sizeof(float);
  return a;
}

template <int G, int KV>
static void launch_tiles_gq(const AttnArgs& A, dim3 grid, bool il, bool phys, hipStream_t s) {
  if (il && phys)
    hipLaunchKernelGGL((attn_tiles_kernel<G, true, true, KV>), grid, dim3(256), 0, s, A);
  else if (il)
    hipLaunchKernelGGL((attn_tiles_kernel<G, true, false, KV>), grid, dim3(256), 0, s, A);
  else if (phys)
    hipLaunchKernelGGL((attn_tiles_kernel<G, false, true, KV>), grid, dim3(256), 0, s, A);
  else
    hipLaunchKernelGGL((attn_tiles_kernel<G, false, false, KV>), grid, dim3(256), 0, s, A);
}

template <int G>
static void launch_tiles_g(const AttnArgs& A, dim3 grid, bool il, bool phys, hipStream_t s) {
  if (A.P.kv == kKvQ8) launch_tiles_gq<G, kKvQ8>(A, grid, il, phys, s);
  else if (A.P.kv == kKvQ4) launch_tiles_gq<G, kKvQ4>(A, grid, il, phys, s);
  else if (A.P.kv == kKvI8) launch_tiles_gq<G, kKvI8>(A, grid, il, phys, s);
  else if (A.P.kv == kKvI4) launch_tiles_gq<G, kKvI4>(A, grid, il, phys, s);
  else launch_tiles_gq<G, kKvFp16>(A, grid, il, phys, s);
}

hipError_t launch_attn_tiles(const AttnArgs& A_in, int batch, bool il, bool sel_phys, hipStream_t s) {
  AttnArgs A = A_in;
  A.P.tl_kind = kTlAttn;
  const int nx = (il ? A.n_il_max : 0) + A.P.topk;
  if (nx <= 0) return hipGetLastError();
  const dim3 grid(nx, A.P.Hkv, batch);
  switch (A.P.g) {
    case 1: launch_tiles_g<1>(A, grid, il, sel_phys, s); break;
    case 2: launch_tiles_g<2>(A, grid, il, sel_phys, s); break;
    case 4: launch_tiles_g<4>(A, grid, il, sel_phys, s); break;
    case 8: launch_tiles_g<8>(A, grid, il, sel_phys, s); break;
    default: launch_tiles_g<16>(A, grid, il, sel_phys, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_merge(const AttnArgs& A, int batch, hipStream_t s) {
  const size_t lds = (size_t)2 * (A.max_parts + 256) * sizeof(float);
  if (lds <= (size_t)kMergeWaveLds) {
    const int n_items = batch * A.P.Hq * (kDim / kMergeChWave);
    hipLaunchKernelGGL(merge_wave_kernel, dim3((n_items + 1) / 2), dim3(128), lds, s, A, n_items);
  } else {
    hipLaunchKernelGGL(merge_kernel, dim3(A.P.Hq * (kDim / kMergeCh), batch), dim3(256), 0, s, A);
  }
  return hipGetLastError();
}

}  // namespace kvs
