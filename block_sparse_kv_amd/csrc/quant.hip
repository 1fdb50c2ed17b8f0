// kvs_quantize_kv: Q8_0, Q4_0 or per-token INT8 records of fp16 K or V tiles.  Q8_0 is the published llama.cpp block
// format that the operator's kv_type list names (KTransformers long-context article, configuration
// list; the instagit page's operator constructor): per token, blocks of 32 channels with scale
// d = max|x| / 127 kept in fp16 and int8 codes round(x / d), ties away from zero.
//
// One workgroup per (listed block, KV head) tile, 256 lanes: lane t takes token t / 2 and channels
// 64 (t % 2) .. +63, i.e. two Q8_0 blocks.  Its 128 bytes of fp16 are contiguous and the wave reads
// 8 KiB in one sweep; codes and scales are written back just as contiguously.  d, 1/d and x * (1/d)
// are IEEE fp32 operations (correctly rounded division), so the codes are exactly those of any fp32
// implementation of the format.
#include "kvs_launch.h"

namespace kvs {

__global__ __launch_bounds__(256) void quantize_q8_kernel(const uint16_t* __restrict__ src,
                                                          const int32_t* __restrict__ ids, int Hkv,
                                                          unsigned char* __restrict__ dst) {
#pragma clang fp contract(off)  // x * (1/d) is rounded before it is rounded to a code
  const int h = blockIdx.x, i = blockIdx.y, t = threadIdx.x;
  const size_t tile = (size_t)ids[i] * Hkv + h;
  const int tok = t >> 1, half = t & 1;
  const uint4* in = reinterpret_cast<const uint4*>(src + tile * kTile + tok * kDim + 64 * half);
  uint4 raw[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) raw[u] = in[u];
  unsigned char* rec = dst + tile * kQ8Record;
  uint32_t codes[16];
  _Float16 sc[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {  // Q8_0 block b of this lane: channels 64 half + 32 b .. +31
    float x[32];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint4 r = raw[4 * b + u];
      const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * u + 2 * e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[e] & 0xFFFFu));
        x[8 * u + 2 * e + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[e] >> 16));
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(x[e]));
    const float d = amax / 127.0f;
    const float inv = d != 0.f ? 1.0f / d : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t word = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float p = x[4 * e + k] * inv;
        const int c = (int)roundf(p);
        word |= (uint32_t)(c & 0xFF) << (8 * k);
      }
      codes[8 * b + e] = word;
    }
    sc[b] = (_Float16)d;
  }
  uint4* co = reinterpret_cast<uint4*>(rec + tok * kDim + 64 * half);
#pragma unroll
  for (int u = 0; u < 4; ++u) co[u] = make_uint4(codes[4 * u], codes[4 * u + 1], codes[4 * u + 2], codes[4 * u + 3]);
  const uint32_t sw = (uint32_t)__builtin_bit_cast(uint16_t, sc[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, sc[1]) << 16);
  *reinterpret_cast<uint32_t*>(rec + kQ8Codes + tok * 8 + 4 * half) = sw;
}

// Q4_0, the format's other block size-32 variant: m = the first value of largest magnitude, d = m / -8,
// codes min(15, trunc(x * (1/d) + 8.5)) (x * (1/d) lies in [-8, 8], so the sum is positive and the
// conversion truncates), all fp32 with IEEE division; d kept in fp16.  Same lane mapping as Q8_0; the
// codes of 8 channels share a word (channel 2i in bits 4i, channel 2i+1 in bits 16+4i).
__global__ __launch_bounds__(256) void quantize_q4_kernel(const uint16_t* __restrict__ src,
                                                          const int32_t* __restrict__ ids, int Hkv,
                                                          unsigned char* __restrict__ dst) {
#pragma clang fp contract(off)
  const int h = blockIdx.x, i = blockIdx.y, t = threadIdx.x;
  const size_t tile = (size_t)ids[i] * Hkv + h;
  const int tok = t >> 1, half = t & 1;
  const uint4* in = reinterpret_cast<const uint4*>(src + tile * kTile + tok * kDim + 64 * half);
  uint4 raw[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) raw[u] = in[u];
  unsigned char* rec = dst + tile * kQ4Record;
  uint32_t words[8];
  _Float16 sc[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float x[32];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint4 r = raw[4 * b + u];
      const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * u + 2 * e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[e] & 0xFFFFu));
        x[8 * u + 2 * e + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[e] >> 16));
      }
    }
    float amax = 0.f, m = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e)
      if (fabsf(x[e]) > amax) { amax = fabsf(x[e]); m = x[e]; }  // the first of the largest
    float d = m / -8.0f;  // -0 for an all-zero block
    // kept as is for the fp16 store: a fused multiply-and-convert adds +0 and would lose the sign of -0
    __asm__ volatile("" : "+v"(d));
    const float inv = d != 0.f ? 1.0f / d : 0.f;
    // x * (1/d) and + 8.5 are two roundings, as the format defines them: no fused multiply-add
    auto code = [&](float v) {
#pragma clang fp contract(off)
      const float p = v * inv;
      return (uint32_t)min(15, (int)(p + 8.5f));
    };
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t word = 0;
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) {
        const uint32_t c0 = code(x[8 * k + 2 * i2]);
        const uint32_t c1 = code(x[8 * k + 2 * i2 + 1]);
        word |= (c0 << (4 * i2)) | (c1 << (16 + 4 * i2));
      }
      words[4 * b + k] = word;
    }
    sc[b] = (_Float16)d;
  }
  uint4* co = reinterpret_cast<uint4*>(rec + tok * (kDim / 2) + 32 * half);
  co[0] = make_uint4(words[0], words[1], words[2], words[3]);
  co[1] = make_uint4(words[4], words[5], words[6], words[7]);
  const uint32_t sw = (uint32_t)__builtin_bit_cast(uint16_t, sc[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, sc[1]) << 16);
  *reinterpret_cast<uint32_t*>(rec + kQ4Codes + tok * 8 + 4 * half) = sw;
}

// INT8 with one scale per token and KV head (the per-token-head int8 cache): s = max|x| / 127 over the
// token's 128 channels, kept in fp32, codes round(x * (1/s)), ties away from zero, as for Q8_0.  Same
// lane mapping; the two lanes of a token combine their maxima with one lane exchange.
__global__ __launch_bounds__(256) void quantize_i8_kernel(const uint16_t* __restrict__ src,
                                                          const int32_t* __restrict__ ids, int Hkv,
                                                          unsigned char* __restrict__ dst) {
#pragma clang fp contract(off)
  const int h = blockIdx.x, i = blockIdx.y, t = threadIdx.x;
  const size_t tile = (size_t)ids[i] * Hkv + h;
  const int tok = t >> 1, half = t & 1;
  const uint4* in = reinterpret_cast<const uint4*>(src + tile * kTile + tok * kDim + 64 * half);
  uint4 raw[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) raw[u] = in[u];
  float x[64];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * u + 2 * e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[e] & 0xFFFFu));
      x[8 * u + 2 * e + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[e] >> 16));
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 64; ++e) amax = fmaxf(amax, fabsf(x[e]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));  // the token's other half
  const float sc = amax / 127.0f;
  const float inv = sc != 0.f ? 1.0f / sc : 0.f;
  uint32_t codes[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float p = x[4 * e + k] * inv;
      word |= (uint32_t)((int)roundf(p) & 0xFF) << (8 * k);
    }
    codes[e] = word;
  }
  unsigned char* rec = dst + tile * kI8Record;
  uint4* co = reinterpret_cast<uint4*>(rec + tok * kDim + 64 * half);
#pragma unroll
  for (int u = 0; u < 4; ++u) co[u] = make_uint4(codes[4 * u], codes[4 * u + 1], codes[4 * u + 2], codes[4 * u + 3]);
  if (half == 0) *reinterpret_cast<float*>(rec + kQ8Codes + tok * 4) = sc;
}

// INT4 with one scale and one zero point per token and KV head (the per-token-head int4 cache, read
// as asymmetric quantization without a rotation): over the token's 128 channels lo = min(0, min x),
// hi = max(0, max x), s = (hi - lo) / 15 kept in fp32, inv = 1 / s, z = clamp(rint(-lo * inv), 0, 15),
// codes clamp(rint(x * inv) + z, 0, 15); rint rounds half to even, every step is an fp32 operation
// (IEEE division, no contraction).  Same lane mapping as Q8_0, the two lanes of a token combining
// their extremes with one lane exchange; the codes are packed as Q4_0's.
__global__ __launch_bounds__(256) void quantize_i4_kernel(const uint16_t* __restrict__ src,
                                                          const int32_t* __restrict__ ids, int Hkv,
                                                          unsigned char* __restrict__ dst) {
#pragma clang fp contract(off)
  const int h = blockIdx.x, i = blockIdx.y, t = threadIdx.x;
  const size_t tile = (size_t)ids[i] * Hkv + h;
  const int tok = t >> 1, half = t & 1;
  const uint4* in = reinterpret_cast<const uint4*>(src + tile * kTile + tok * kDim + 64 * half);
  uint4 raw[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) raw[u] = in[u];
  float x[64];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * u + 2 * e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[e] & 0xFFFFu));
      x[8 * u + 2 * e + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[e] >> 16));
    }
  }
  float lo = 0.f, hi = 0.f;  // the range holds 0
#pragma unroll
  for (int e = 0; e < 64; ++e) {
    lo = fminf(lo, x[e]);
    hi = fmaxf(hi, x[e]);
  }
  lo = fminf(lo, __shfl_xor(lo, 1, 64));  // the token's other half
  hi = fmaxf(hi, __shfl_xor(hi, 1, 64));
  const float sc = (hi - lo) / 15.0f;
  const float inv = sc != 0.f ? 1.0f / sc : 0.f;
  const float nlo = -lo;
  const int z = sc != 0.f ? min(15, max(0, (int)rintf(nlo * inv))) : 0;
  auto code = [&](float v) {
    const float p = v * inv;
    return (uint32_t)min(15, max(0, (int)rintf(p) + z));
  };
  uint32_t words[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    uint32_t word = 0;
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
      const uint32_t c0 = code(x[8 * k + 2 * i2]);
      const uint32_t c1 = code(x[8 * k + 2 * i2 + 1]);
      word |= (c0 << (4 * i2)) | (c1 << (16 + 4 * i2));
    }
    words[k] = word;
  }
  unsigned char* rec = dst + tile * kI4Record;
  uint4* co = reinterpret_cast<uint4*>(rec + tok * (kDim / 2) + 32 * half);
  co[0] = make_uint4(words[0], words[1], words[2], words[3]);
  co[1] = make_uint4(words[4], words[5], words[6], words[7]);
  if (half == 0) {
    *reinterpret_cast<float*>(rec + kI4Scales + tok * 4) = sc;
    rec[kI4Zeros + tok] = (unsigned char)z;
  }
}

hipError_t launch_quantize_q8(const Params& P, const void* src, const int32_t* ids, int n, void* dst,
                              hipStream_t s) {
  if (P.kv == kKvI4)
    hipLaunchKernelGGL(quantize_i4_kernel, dim3(P.Hkv, n), dim3(256), 0, s,
                       static_cast<const uint16_t*>(src), ids, P.Hkv, static_cast<unsigned char*>(dst));
  else if (P.kv == kKvI8)
    hipLaunchKernelGGL(quantize_i8_kernel, dim3(P.Hkv, n), dim3(256), 0, s,
                       static_cast<const uint16_t*>(src), ids, P.Hkv, static_cast<unsigned char*>(dst));
  else if (P.kv == kKvQ4)
    hipLaunchKernelGGL(quantize_q4_kernel, dim3(P.Hkv, n), dim3(256), 0, s,
                       static_cast<const uint16_t*>(src), ids, P.Hkv, static_cast<unsigned char*>(dst));
  else
    hipLaunchKernelGGL(quantize_q8_kernel, dim3(P.Hkv, n), dim3(256), 0, s,
                       static_cast<const uint16_t*>(src), ids, P.Hkv, static_cast<unsigned char*>(dst));
  return hipGetLastError();
}

}  // namespace kvs
