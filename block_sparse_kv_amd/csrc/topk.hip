// kvs_topk_blocks kernel: per (sequence, selection group) keep the top-k Context blocks
// (KTransformers long-context sparse attention, lmnt.cn: §3.1 select the top-k blocks by score;
// §4.5 second_block_count).  Ties go to the lower block index; the output is in ascending order.
//
// One workgroup of 1024 lanes per (sequence, group).  Scores become order-preserving 32-bit keys
// (+0 and -0 share one key) staged in LDS; an MSB-first radix select (4 passes of 8 bits, LDS
// histogram, one-wave suffix scan) finds the k-th largest key T and how many keys equal to T are
// needed.  A workgroup-wide scan over contiguous per-lane index ranges then keeps every key > T and the
// lowest-indexed keys == T, and a second scan gives each kept block its slot in ascending order.
#include "kvs_device.h"
#include "kvs_launch.h"

namespace kvs {

constexpr int kTopkThreads = 1024;
constexpr int kTopkLdsKeys = 16384;  // 64 KiB of keys: candidates beyond this read global memory

__device__ inline uint32_t order_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if (f == 0.f) u = 0u;  // one key for +0 and -0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the workgroup (1024 lanes = 16 waves); also returns the total.
__device__ inline int block_exclusive_scan(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wave_tot[w] = x;
  __syncthreads();
  if (w == 0) {
    int tv = lane < 16 ? wave_tot[lane] : 0;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int y = __shfl_up(tv, d, 64);
      if (lane >= d) tv += y;
    }
    if (lane < 16) wave_tot[16 + lane] = tv;  // inclusive wave prefix
  }
  __syncthreads();
  const int before = (w == 0 ? 0 : wave_tot[16 + w - 1]) + x - v;
  total = wave_tot[16 + 15];
  __syncthreads();
  return before;
}

template <bool IN_LDS>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(Params P, const float* __restrict__ scores,
                                                            const int32_t* __restrict__ seq_lens,
                                                            int max_blocks, int32_t* __restrict__ sel,
                                                            int32_t* __restrict__ sel_count) {
  const int grp = blockIdx.x, seq = blockIdx.y, tid = threadIdx.x;
  const int L = seq_lens[seq];
  const Regions rg = regions_of(L, P.initial_len, P.local_len);
  const int n = rg.cand_hi - rg.cand_lo;
  const int k = min(P.topk, n);
  const size_t row_id = (size_t)seq * P.G + grp;
  const float* row = scores + row_id * max_blocks + rg.cand_lo;
  int32_t* out = sel + row_id * P.topk;
  if (tid == 0) sel_count[row_id] = k;
  for (int i = k + tid; i < P.topk; i += kTopkThreads) out[i] = -1;
  if (k == 0) return;
  if (k == n) {
    for (int i = tid; i < n; i += kTopkThreads) out[i] = rg.cand_lo + i;
    return;
  }

  __shared__ uint32_t lkeys[IN_LDS ? kTopkLdsKeys : 1];
  __shared__ int hist[256];
  __shared__ int bcast[2];
  __shared__ int wave_tot[32];
  if constexpr (IN_LDS)
    for (int i = tid; i < n; i += kTopkThreads) lkeys[i] = order_key(row[i]);
  auto key = [&](int i) -> uint32_t {
    if constexpr (IN_LDS) return lkeys[i];
    else return order_key(row[i]);
  };

  uint32_t prefix = 0, pmask = 0;
  int rem = k;  // still to take among keys matching the prefix, counted from the top
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kTopkThreads) {
      const uint32_t u = key(i);
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255], 1);
    }
    __syncthreads();
    if (tid < 64) {  // lane l owns digits 4l..4l+3; suffix sums from the high digits
      const int c0 = hist[4 * tid], c1 = hist[4 * tid + 1], c2 = hist[4 * tid + 2], c3 = hist[4 * tid + 3];
      const int own = c0 + c1 + c2 + c3;
      int suf = own;  // inclusive suffix over lanes >= tid
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_down(suf, d, 64);
        if (tid + d < 64) suf += y;
      }
      const int above_lane = suf - own;  // count with digit > 4*tid+3
      if (above_lane < rem && suf >= rem) {
        // walk this lane's digits from the top: 4l+3, 4l+2, 4l+1, 4l
        int digit, above = above_lane;
        if (above + c3 >= rem) digit = 4 * tid + 3;
        else if ((above += c3) + c2 >= rem) digit = 4 * tid + 2;
        else if ((above += c2) + c1 >= rem) digit = 4 * tid + 1;
        else { above += c1; digit = 4 * tid; }
        bcast[0] = digit;
        bcast[1] = above;
      }
    }
    __syncthreads();
    const int digit = bcast[0];
    rem -= bcast[1];
    prefix |= (uint32_t)digit << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t T = prefix;  // the k-th largest key; take `rem` of the keys equal to T

  const int per = (n + kTopkThreads - 1) / kTopkThreads;
  const int i0 = min(n, tid * per), i1 = min(n, i0 + per);
  int n_eq = 0;
  for (int i = i0; i < i1; ++i) n_eq += key(i) == T;
  int tot;
  int eq_rank = block_exclusive_scan(n_eq, wave_tot, tot);
  int n_keep = 0;
  {
    int r = eq_rank;
    for (int i = i0; i < i1; ++i) {
      const uint32_t u = key(i);
      if (u > T) ++n_keep;
      else if (u == T) { n_keep += r < rem; ++r; }
    }
  }
  int pos = block_exclusive_scan(n_keep, wave_tot, tot);
  int r = eq_rank;
  for (int i = i0; i < i1; ++i) {
    const uint32_t u = key(i);
    bool keep = u > T;
    if (u == T) { keep = r < rem; ++r; }
    if (keep && pos < k) out[pos++] = rg.cand_lo + i;
  }
}

hipError_t launch_topk(const Params& P, const float* scores, const int32_t* seq_lens, int batch,
                       int max_blocks, int32_t* sel, int32_t* sel_count, hipStream_t s) {
  const dim3 grid(P.G, batch), block(kTopkThreads);
  if (max_blocks <= kTopkLdsKeys)
    hipLaunchKernelGGL(topk_kernel<true>, grid, block, 0, s, P, scores, seq_lens, max_blocks, sel, sel_count);
  else
    hipLaunchKernelGGL(topk_kernel<false>, grid, block, 0, s, P, scores, seq_lens, max_blocks, sel, sel_count);
  return hipGetLastError();
}

}  // namespace kvs
