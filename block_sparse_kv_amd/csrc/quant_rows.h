// Cached values of one token row of a quantized K/V record, 8 channels at a time, in fp32: the
// value a record stands for (Q8_0: scale * code, Q4_0: scale * (code - 8), both exact in fp32; INT8
// per token and head: the fp32 product of the token's scale and the code; INT4 per token and head:
// the fp32 product of the token's scale and code - zero point).
#pragma once

#include "kvs_device.h"

namespace kvs {

// 8 cached values of a Q8_0 record: channels 8c..8c+7 of token `tok` (scale * code, exact in fp32).
__device__ inline void q8_row8(const unsigned char* rec, int tok, int c, float f[8]) {
  const uint2 cw = *reinterpret_cast<const uint2*>(rec + tok * kDim + c * 8);
  const float d = (float)__builtin_bit_cast(_Float16, *reinterpret_cast<const uint16_t*>(
                      rec + kQ8Codes + tok * (kDim / kQ8Group) * 2 + (c * 8 / kQ8Group) * 2));
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t w = e < 4 ? cw.x : cw.y;
    f[e] = (float)(int)(signed char)((w >> (8 * (e & 3))) & 0xFF) * d;
  }
}

// 8 cached values of a Q4_0 record: channels 8c..8c+7 of token `tok` (word c of its row), d * (code - 8).
__device__ inline void q4_row8(const unsigned char* rec, int tok, int c, float f[8]) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(rec + tok * (kDim / 2) + c * 4);
  const float d = (float)__builtin_bit_cast(_Float16, *reinterpret_cast<const uint16_t*>(
                      rec + kQ4Codes + tok * (kDim / kQ8Group) * 2 + (c * 8 / kQ8Group) * 2));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = (float)((int)((w >> (4 * i)) & 0xF) - 8) * d;
    f[2 * i + 1] = (float)((int)((w >> (16 + 4 * i)) & 0xF) - 8) * d;
  }
}

// 8 cached values of an INT8 per-token-head record: channels 8c..8c+7 of token `tok`, fp32(s * code).
__device__ inline void i8_row8(const unsigned char* rec, int tok, int c, float f[8]) {
  const uint2 cw = *reinterpret_cast<const uint2*>(rec + tok * kDim + c * 8);
  const float s = *reinterpret_cast<const float*>(rec + kQ8Codes + tok * 4);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t w = e < 4 ? cw.x : cw.y;
    f[e] = (float)(int)(signed char)((w >> (8 * (e & 3))) & 0xFF) * s;
    keep_fp32(f[e]);
  }
}

// 8 cached values of an INT4 per-token-head record: channels 8c..8c+7 of token `tok` (word c of its
// row, Q4_0's layout), fp32(s * (code - z)).
__device__ inline void i4_row8(const unsigned char* rec, int tok, int c, float f[8]) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(rec + tok * (kDim / 2) + c * 4);
  const float s = *reinterpret_cast<const float*>(rec + kI4Scales + tok * 4);
  const int z = rec[kI4Zeros + tok];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = (float)((int)((w >> (4 * i)) & 0xF) - z) * s;
    f[2 * i + 1] = (float)((int)((w >> (16 + 4 * i)) & 0xF) - z) * s;
    keep_fp32(f[2 * i]);
    keep_fp32(f[2 * i + 1]);
  }
}

}  // namespace kvs
