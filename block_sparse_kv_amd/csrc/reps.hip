// kvs_build_reps kernels: representative keys of full 128-token blocks
// (KTransformers long-context sparse attention, lmnt.cn, §4.3 rep methods; §3.1 Quest's
// channel-wise min/max "Reduced Keys").
//
// One workgroup (256 lanes) per (listed block, KV head) tile of 128 x 128 fp16 = 32 KiB.  Lane t reads
// channels 8*(t%16)..+8 of tokens t/16 + 16*i (i = 0..7) with 128-bit loads: each wave-wide load is
// 4 whole token rows, 1 KiB contiguous.  Per-lane partials are folded across the 4 rows of a wave
// with lane shuffles and across the 4 waves through LDS.  The kernel streams K once (HBM-bound).
// A Q8_0 cache (kv_type; the llama.cpp block format) is read the same way, 8 codes and the scale of
// their 32-channel block per token; scale * code is exact in fp32, and the reps are rounded to fp16
// once, at the store.  Q4_0 and the per-token INT8 and INT4 caches likewise (INT8: the cached value is
// the fp32 product of the token's scale and the code; INT4: of the scale and the code less the token's
// zero point).
#include "kvs_device.h"
#include "kvs_launch.h"
#include "quant_rows.h"

namespace kvs {

template <int METHOD, int KV>
__global__ __launch_bounds__(256) void build_reps_kernel(const void* __restrict__ k_pool,
                                                         const int32_t* __restrict__ ids, int Hkv,
                                                         int rep_num, void* __restrict__ rep_pool) {
  const int h = blockIdx.y;
  const size_t p = (size_t)ids[blockIdx.x];
  const uint16_t* tile = static_cast<const uint16_t*>(k_pool) + (p * Hkv + h) * kTile;
  const unsigned char* rec = static_cast<const unsigned char*>(k_pool) +
                             (p * Hkv + h) * (size_t)(KV == kKvQ4 ? kQ4Record : KV == kKvI8 ? kI8Record : KV == kKvI4 ? kI4Record : kQ8Record);
  constexpr bool Q8 = KV != kKvFp16;  // a quantized record
  const int t = threadIdx.x, c = t & 15, r = t >> 4;

  if constexpr (METHOD == kFix) {  // rows 0, s, 2s, ... (fp16: copied verbatim)
    const int stride = kBlock / rep_num;
    uint16_t* out = static_cast<uint16_t*>(rep_pool) + (p * Hkv + h) * (size_t)rep_num * kDim;
    for (int rr = r; rr < rep_num; rr += 16) {
      if constexpr (Q8) {
        float f[8];
        if constexpr (KV == kKvQ4) q4_row8(rec, rr * stride, c, f);
        else if constexpr (KV == kKvI8) i8_row8(rec, rr * stride, c, f);
        else if constexpr (KV == kKvI4) i4_row8(rec, rr * stride, c, f);
        else q8_row8(rec, rr * stride, c, f);
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (uint32_t)f2h_bits(f[2 * e]) | ((uint32_t)f2h_bits(f[2 * e + 1]) << 16);
        *reinterpret_cast<uint4*>(out + rr * kDim + c * 8) = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
        *reinterpret_cast<uint4*>(out + rr * kDim + c * 8) =
            *reinterpret_cast<const uint4*>(tile + (size_t)(rr * stride) * kDim + c * 8);
      }
    }
    return;
  } else {
    uint4 raw[8];
    if constexpr (!Q8) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        raw[i] = ld_stream16(tile + (size_t)(r + 16 * i) * kDim + c * 8);
    }
    float a[8], b[8];  // Quest: min, max.  Max: -, max.  Mean: sum, -
#pragma unroll
    for (int e = 0; e < 8; ++e) { a[e] = METHOD == kMean ? 0.f : INFINITY; b[e] = -INFINITY; }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float f[8];
      if constexpr (KV == kKvQ4) q4_row8(rec, r + 16 * i, c, f);
      else if constexpr (KV == kKvQ8) q8_row8(rec, r + 16 * i, c, f);
      else if constexpr (KV == kKvI8) i8_row8(rec, r + 16 * i, c, f);
      else if constexpr (KV == kKvI4) i4_row8(rec, r + 16 * i, c, f);
      else unpack8(raw[i], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (METHOD == kMean) a[e] += f[e];
        if (METHOD == kQuest) a[e] = fminf(a[e], f[e]);
        if (METHOD != kMean) b[e] = fmaxf(b[e], f[e]);
      }
    }
    // fold the 4 rows of this wave (lanes l, l^16, l^32, l^48 share the channels)
#pragma unroll
    for (int m = 16; m <= 32; m <<= 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ao = shfl_xor_f(a[e], m), bo = shfl_xor_f(b[e], m);
        if (METHOD == kMean) a[e] += ao;
        if (METHOD == kQuest) a[e] = fminf(a[e], ao);
        if (METHOD != kMean) b[e] = fmaxf(b[e], bo);
      }
    }
    __shared__ float sa[4][kDim], sb[4][kDim];
    const int w = t >> 6;
    if ((t & 63) < 16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) { sa[w][c * 8 + e] = a[e]; sb[w][c * 8 + e] = b[e]; }
    }
    __syncthreads();
    if (t < kDim) {
      if constexpr (METHOD == kMean) {
        const float s = ((sa[0][t] + sa[1][t]) + sa[2][t]) + sa[3][t];
        float* out = static_cast<float*>(rep_pool) + (p * Hkv + h) * kDim;
        out[t] = s * (1.0f / kBlock);  // power-of-two scale: exact
      } else {
        uint16_t* out = static_cast<uint16_t*>(rep_pool) + (p * Hkv + h) * (size_t)(METHOD == kQuest ? 2 : 1) * kDim;
        const float mx = fmaxf(fmaxf(sb[0][t], sb[1][t]), fmaxf(sb[2][t], sb[3][t]));
        if constexpr (METHOD == kQuest) {
          const float mn = fminf(fminf(sa[0][t], sa[1][t]), fminf(sa[2][t], sa[3][t]));
          out[t] = f2h_bits(mn);
          out[kDim + t] = f2h_bits(mx);
        } else {
          out[t] = f2h_bits(mx);
        }
      }
    }
  }
}

template <int KV>
static void launch_reps_q(const Params& P, dim3 grid, const void* kp, const int32_t* ids, int rep_num,
                          void* rep_pool, hipStream_t s) {
  const dim3 block(256);
  switch (P.method) {
    case kQuest: hipLaunchKernelGGL((build_reps_kernel<kQuest, KV>), grid, block, 0, s, kp, ids, P.Hkv, rep_num, rep_pool); break;
    case kMax:   hipLaunchKernelGGL((build_reps_kernel<kMax, KV>), grid, block, 0, s, kp, ids, P.Hkv, rep_num, rep_pool); break;
    case kMean:  hipLaunchKernelGGL((build_reps_kernel<kMean, KV>), grid, block, 0, s, kp, ids, P.Hkv, rep_num, rep_pool); break;
    default:     hipLaunchKernelGGL((build_reps_kernel<kFix, KV>), grid, block, 0, s, kp, ids, P.Hkv, rep_num, rep_pool); break;
  }
}

hipError_t launch_build_reps(const Params& P, const void* k_pool, const int32_t* ids, int n,
                             int rep_num, void* rep_pool, hipStream_t s) {
  const dim3 grid(n, P.Hkv);
  if (P.kv == kKvQ8) launch_reps_q<kKvQ8>(P, grid, k_pool, ids, rep_num, rep_pool, s);
  else if (P.kv == kKvQ4) launch_reps_q<kKvQ4>(P, grid, k_pool, ids, rep_num, rep_pool, s);
  else if (P.kv == kKvI8) launch_reps_q<kKvI8>(P, grid, k_pool, ids, rep_num, rep_pool, s);
  else if (P.kv == kKvI4) launch_reps_q<kKvI4>(P, grid, k_pool, ids, rep_num, rep_pool, s);
  else launch_reps_q<kKvFp16>(P, grid, k_pool, ids, rep_num, rep_pool, s);
  return hipGetLastError();
}

}  // namespace kvs
