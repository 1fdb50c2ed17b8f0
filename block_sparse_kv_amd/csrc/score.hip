// kvs_score_blocks kernel: block relevance against the current query
// (KTransformers long-context sparse attention, lmnt.cn: §3.1 Quest upper bound
// sum_c max(q_c*kmax_c, q_c*kmin_c); §4.3 similarity with the reps; §4.5 SEPARATE / SHARED).
//
// Lane layout: 16 lanes (one DPP row) per (logical block, KV head); lane c owns channels 8c..8c+7 and
// keeps the matching slice of the g query heads of its KV head in registers.  A workgroup of 256
// lanes covers 16/Hkv blocks x Hkv heads.  Reps are read with 128-bit loads: one row of 16 lanes reads
// one 256-byte fp16 rep row.  For the linear reps (Max, Mean, Fix) the g query heads are summed first,
// since sum_j q_j.rep = (sum_j q_j).rep; Quest is per head (the max is not linear).
#include "kvs_device.h"
#include "kvs_launch.h"

namespace kvs {

template <int G, int METHOD, int MODE>
__global__ __launch_bounds__(256) void score_kernel(Params P, const uint16_t* __restrict__ q,
                                                    const void* __restrict__ rep_pool,
                                                    const int32_t* __restrict__ table, int max_blocks,
                                                    const int32_t* __restrict__ seq_lens,
                                                    float* __restrict__ scores) {
  const int seq = blockIdx.y;
  const int Hkv = P.Hkv;
  const int t = threadIdx.x, c = t & 15;
  const int h = (t >> 4) % Hkv;
  const int bpw = 16 / Hkv;  // blocks per workgroup
  const int slot = (t >> 4) / Hkv;
  const int b = blockIdx.x * bpw + slot;
  const int L = seq_lens[seq];
  const Regions rg = regions_of(L, P.initial_len, P.local_len);
  const bool cand = b >= rg.cand_lo && b < rg.cand_hi;

  float acc = 0.f;
  if (cand) {
    const size_t phys = (size_t)table[(size_t)seq * max_blocks + b];
    const uint16_t* qh = q + ((size_t)seq * P.Hq + (size_t)h * G) * kDim + c * 8;
    float qf[G][8];
#pragma unroll
    for (int j = 0; j < G; ++j) unpack8(*reinterpret_cast<const uint4*>(qh + j * kDim), qf[j]);
    if constexpr (METHOD == kQuest) {
      const uint16_t* rp = static_cast<const uint16_t*>(rep_pool) + (phys * Hkv + h) * 2 * kDim + c * 8;
      float kmin[8], kmax[8];
      unpack8(*reinterpret_cast<const uint4*>(rp), kmin);
      unpack8(*reinterpret_cast<const uint4*>(rp + kDim), kmax);
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += fmaxf(qf[j][e] * kmax[e], qf[j][e] * kmin[e]);
    } else {
      float qs[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qs[e] = 0.f;
#pragma unroll
        for (int j = 0; j < G; ++j) qs[e] += qf[j][e];
      }
      float rs[8];
      if constexpr (METHOD == kMean) {
        const float* rp = static_cast<const float*>(rep_pool) + (phys * Hkv + h) * kDim + c * 8;
        const float4 x0 = *reinterpret_cast<const float4*>(rp);
        const float4 x1 = *reinterpret_cast<const float4*>(rp + 4);
        rs[0] = x0.x; rs[1] = x0.y; rs[2] = x0.z; rs[3] = x0.w;
        rs[4] = x1.x; rs[5] = x1.y; rs[6] = x1.z; rs[7] = x1.w;
      } else {
        const int R = P.R;
        const uint16_t* rp = static_cast<const uint16_t*>(rep_pool) + (phys * Hkv + h) * (size_t)R * kDim + c * 8;
        unpack8(*reinterpret_cast<const uint4*>(rp), rs);
        for (int r = 1; r < R; ++r) {  // Fix: the sum of the rep rows, then one dot
          float f[8];
          unpack8(*reinterpret_cast<const uint4*>(rp + (size_t)r * kDim), f);
#pragma unroll
          for (int e = 0; e < 8; ++e) rs[e] += f[e];
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += qs[e] * rs[e];
    }
  }
  acc = row_sum16(acc);

  if constexpr (MODE == kSeparate) {
    if (c == 0 && b < max_blocks)
      scores[((size_t)seq * Hkv + h) * max_blocks + b] = cand ? acc : -INFINITY;
  } else {
    __shared__ float part[16];  // [slot][h], slot * Hkv + h < 16
    if (c == 0) part[slot * Hkv + h] = acc;
    __syncthreads();
    if (c == 0 && h == 0 && b < max_blocks) {
      float s = 0.f;
      for (int hh = 0; hh < Hkv; ++hh) s += part[slot * Hkv + hh];
      scores[(size_t)seq * max_blocks + b] = cand ? s : -INFINITY;
    }
  }
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
  const int bpw = 16 / P.Hkv;
  const dim3 grid((max_blocks + bpw - 1) / bpw, batch);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  switch (P.g) {
    case 1: launch_score_g<1>(P, grid, s, qq, rep_pool, table, max_blocks, seq_lens, scores); break;
    case 2: launch_score_g<2>(P, grid, s, qq, rep_pool, table, max_blocks, seq_lens, scores); break;
    case 4: launch_score_g<4>(P, grid, s, qq, rep_pool, table, max_blocks, seq_lens, scores); break;
    default: launch_score_g<8>(P, grid, s, qq, rep_pool, table, max_blocks, seq_lens, scores); break;
  }
  return hipGetLastError();
}

}  // namespace kvs
