// kvs_sparse_decode_attn kernels (standalone attention over a given selection):
//  * tile plan: per (sequence, selection group) the physical ids of the attended tiles in order --
//    Initial tiles, the selected tiles, the Local tiles -- and their count;
//  * split attention: workgroup (split, h, seq) runs attn_partial (attn_core.h) over `tps`
//    consecutive tiles of the list;
//  * merge: workgroup (h, seq) combines the splits of the g query heads of KV head h by
//    log-sum-exp (merge_heads).
#include "attn_core.h"
#include "kvs_launch.h"

namespace kvs {

__global__ __launch_bounds__(128) void tile_plan_kernel(Params P, const int32_t* __restrict__ table,
                                                        int max_blocks, const int32_t* __restrict__ seq_lens,
                                                        const int32_t* __restrict__ sel,
                                                        const int32_t* __restrict__ sel_count, int maxT,
                                                        int32_t* __restrict__ tiles, int32_t* __restrict__ ntiles) {
  const int grp = blockIdx.x, seq = blockIdx.y;
  const int L = seq_lens[seq];
  const size_t grow = (size_t)seq * P.G + grp;
  const Regions rg = regions_of(L, P.initial_len, P.local_len);
  const int k_sel = L > rg.init_end ? sel_count[grow] : 0;
  const TileList tl = tiles_of(L, P, k_sel);
  const int nT = min(tl.count(), maxT);
  const int32_t* trow = table + (size_t)seq * max_blocks;
  const int32_t* srow = sel + grow * P.topk;
  int32_t* out = tiles + grow * maxT;
  for (int t = threadIdx.x; t < maxT; t += blockDim.x) {
    int phys = -1;
    if (t < nT) {
      int lb;
      if (t < tl.nI) lb = t;
      else if (t < tl.nI + tl.k) lb = srow[t - tl.nI];
      else lb = tl.loc_b0 + (t - tl.nI - tl.k);
      phys = trow[lb];
    }
    out[t] = phys;
  }
  if (threadIdx.x == 0) ntiles[grow] = nT;
}

template <int G>
__global__ __launch_bounds__(256) void attn_split_kernel(
    Params P, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ ntiles, int maxT, int tps,
    int n_splits, float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kAttnLdsBytes];
  const int split = blockIdx.x, h = blockIdx.y, seq = blockIdx.z;
  const size_t grow = (size_t)seq * P.G + (P.mode == kSeparate ? h : 0);
  const int nT = ntiles[grow];
  const int t0 = split * tps;
  if (t0 >= nT) return;
  const int n = min(tps, nT - t0);
  const int L = seq_lens[seq];
  const int last_ntok = L - kBlock * ((L - 1) / kBlock);  // tokens in the list's last tile
  const int32_t* trow = tiles + grow * maxT + t0;
  const size_t head0 = (size_t)seq * P.Hq + (size_t)h * G;
  attn_partial<G, false>(P, q + head0 * kDim, k_pool, v_pool, h, n,
                  [&](int i) -> int2 { return make_int2(trow[i], t0 + i == nT - 1 ? last_ntok : kBlock); },
                  part_o + head0 * n_splits * kDim, part_ml + head0 * n_splits * 2, n_splits, split,
                  smem);
}

template <int G>
__global__ __launch_bounds__(256) void attn_merge_kernel(Params P, const int32_t* __restrict__ ntiles,
                                                         int tps, int n_splits,
                                                         const float* __restrict__ part_o,
                                                         const float* __restrict__ part_ml,
                                                         float* __restrict__ out) {
  __shared__ float lds[kMergeLdsFloats];
  const int h = blockIdx.x, seq = blockIdx.y;
  const int nT = ntiles[(size_t)seq * P.G + (P.mode == kSeparate ? h : 0)];
  const int ns = (nT + tps - 1) / tps;
  const size_t head0 = (size_t)seq * P.Hq + (size_t)h * G;
  merge_heads<G, false>(part_o + head0 * n_splits * kDim, part_ml + head0 * n_splits * 2, n_splits, ns,
                        out + head0 * kDim, lds);
}

AttnPlan attn_plan(const Params& P, int batch, int max_blocks) {
  const int nI = (P.initial_len + kBlock - 1) / kBlock;
  const int nLoc = (P.local_len + 2 * kBlock - 2) / kBlock;
  long maxT = (long)nI + P.topk + nLoc;
  if (maxT > max_blocks) maxT = max_blocks;
  if (maxT < 1) maxT = 1;
  const long total = (long)batch * P.Hkv * maxT;
  long tps = total / 1024;
  if (tps < 1) tps = 1;
  if (tps < (maxT + kMaxParts - 1) / kMaxParts) tps = (maxT + kMaxParts - 1) / kMaxParts;
  if (tps > kMaxItemTiles) tps = kMaxItemTiles;
  AttnPlan a;
  a.maxT = (int)maxT;
  a.tps = (int)tps;
  a.n_splits = (int)((maxT + tps - 1) / tps);
  a.part_o_bytes = (size_t)batch * P.Hq * a.n_splits * kDim * sizeof(float);
  a.part_ml_bytes = (size_t)batch * P.Hq * a.n_splits * 2 * sizeof(float);
  a.tiles_bytes = (size_t)batch * P.G * maxT * sizeof(int32_t);
  a.ntiles_bytes = (size_t)batch * P.G * sizeof(int32_t);
  return a;
}

hipError_t launch_tile_plan(const Params& P, const AttnPlan& A, const int32_t* table, int max_blocks,
                            const int32_t* seq_lens, int batch, const int32_t* sel,
                            const int32_t* sel_count, int32_t* tiles, int32_t* ntiles, hipStream_t s) {
  hipLaunchKernelGGL(tile_plan_kernel, dim3(P.G, batch), dim3(128), 0, s, P, table, max_blocks,
                     seq_lens, sel, sel_count, A.maxT, tiles, ntiles);
  return hipGetLastError();
}

hipError_t launch_attn(const Params& P, const AttnPlan& A, const void* q, const void* k_pool,
                       const void* v_pool, const int32_t* seq_lens, int batch, const int32_t* tiles,
                       const int32_t* ntiles, float* out, float* part_o, float* part_ml,
                       hipStream_t s) {
  const dim3 grid(A.n_splits, P.Hkv, batch), block(256), mgrid(P.Hkv, batch);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kp = static_cast<const uint16_t*>(k_pool);
  const uint16_t* vp = static_cast<const uint16_t*>(v_pool);
#define KVS_ATTN(GG)                                                                                  \
  hipLaunchKernelGGL(attn_split_kernel<GG>, grid, block, 0, s, P, qq, kp, vp, seq_lens, tiles, ntiles,  \
                     A.maxT, A.tps, A.n_splits, part_o, part_ml);                                      \
  hipLaunchKernelGGL(attn_merge_kernel<GG>, mgrid, block, 0, s, P, ntiles, A.tps, A.n_splits, part_o, \
                     part_ml, out)
  switch (P.g) {
    case 1: KVS_ATTN(1); break;
    case 2: KVS_ATTN(2); break;
    case 4: KVS_ATTN(4); break;
    case 8: KVS_ATTN(8); break;
    default: KVS_ATTN(16); break;
  }
#undef KVS_ATTN
  return hipGetLastError();
}

}  // namespace kvs
