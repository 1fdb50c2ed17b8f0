// Exact attention over one K/V tile on the matrix cores, for one workgroup of 256 lanes, and the
// log-sum-exp merge of the per-tile partials (used by kvs_sparse_decode_attn and kvs_decode_step).
// KTransformers long-context sparse attention (lmnt.cn): §4.2 Initial and Local are always attended
// with the selected Context blocks in between; §4.6 attn(query, kvcache_after_retrieval) with logits
// scaled by 1/sqrt(head_dim).
//
// Every attended (block, KV head) tile is one workgroup: its 64 KiB of K and V are requested at once,
// and with 4 such workgroups per CU (at most 128 registers and 36 KiB of LDS each) a whole decode
// step's tiles are in flight together, which is what an HBM-bound gather needs.  A tile covers all
// g <= 16 query heads of its KV head, padded to the 16 rows of v_mfma_f32_16x16x32_f16.  Each of the
// 4 waves owns 32 token rows:
//   S = K Q^T: the A operand is lane l: token l%16, channels 8*(l/16)..+8 of a 32-channel chunk.
//     fp16 K, and the 128-B code rows of Q8_0 and INT8 K, pass through LDS, loaded by whole token
//     rows (1 KiB per load) and read back in that layout; Q4_0 and INT4 K codes (64-B rows, so 16
//     rows are 1 KiB anyway) come straight from HBM in it.  Q^T is a register-resident B operand.
//   softmax in the exp2 domain per head (the 4 lanes holding one head combine with two shuffles); P is
//     rounded to fp16 and the row sums use the rounded values.
//   O = P V: P is already in the A-operand layout (k-slot 8*(l/16)+e holds token 16*(e/4)+4*(l/16)+e%4).
//     V passes through LDS, token rows padded to 288 B, and reaches the B-operand layout (8 tokens of
//     one channel per lane) through ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives
//     element i%4 of the 8-byte chunks addressed by lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4, so
//     lane s of the group points at channels 16nn + 4(s%4) .. +3 of token row s/4 of a 4-token chunk.
// The 4 waves fold through LDS into one partial (max, sum, unnormalised output) per query head.
#pragma once

#include "kvs_device.h"

namespace kvs {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ inline f32x4_t ld_stream16f(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
}

constexpr int kNtLoad = 2;  // cache-policy operand of the K buffer loads: non-temporal, as ld_stream16
constexpr int kVRow = 288;                      // bytes per staged V token row (256 + 32 bank skew)
constexpr int kVChunk = 4 * kVRow;              // 4 token rows
constexpr int kWaveVBytes = 8 * kVChunk;        // V staging per wave (32 tokens)
constexpr int kAttnLdsBytes = 4 * kWaveVBytes;  // also >= the fold buffers for G <= 16
static_assert(kBlock / 4 * kDim * 2 <= kWaveVBytes, "a wave's K rows fit its V staging area");

typedef short v4s_t __attribute__((ext_vector_type(4)));
__device__ inline v4s_t lds_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(p));
}

// Partial of query heads h*G .. h*G+G-1 over one tile (physical block `phys`, its first `ntok`
// tokens, 0 <= ntok <= 128).  Writes part_o[j * n_parts + part][128] and
// part_ml[(j * n_parts + part) * 2 + {0: max, 1: sum}] for j < G (arrays already offset to the first
// query head of h).
//
// The workgroup may be a 256-lane part of a larger one (smem then points at the part's area): every
// part runs the same barriers.  ntok == 0 gives an empty partial (max -inf); with
// store == false nothing is written.
// 4 Q8_0 codes (the bytes of w, lowest first) times the fp16 scale d, as 4 fp16 values in 2 words:
// fp16(code * d), rounded once.  A code c becomes the fp16 1024 + (c + 128) by placing the biased byte
// under the exponent pattern 0x64 (v_perm_b32), which the packed subtraction of 1152 turns into c
// exactly; one packed multiply then applies d.
typedef _Float16 half2v_t __attribute__((ext_vector_type(2)));
__device__ inline uint2 q8_dq4(uint32_t w, half2v_t d2) {
  const uint32_t u = w ^ 0x80808080u;
  const half2v_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  const half2v_t lo = (__builtin_bit_cast(half2v_t, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) - bias) * d2;
  const half2v_t hi = (__builtin_bit_cast(half2v_t, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) - bias) * d2;
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}
// 8 codes (w0 then w1) with the fp16 scale in the low half of sc.
__device__ inline uint4 q8_dq8(uint32_t w0, uint32_t w1, uint32_t sc) {
  const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)(sc & 0xFFFFu));
  const half2v_t d2 = {d, d};
  const uint2 a = q8_dq4(w0, d2), b = q8_dq4(w1, d2);
  return make_uint4(a.x, a.y, b.x, b.y);
}

// 8 Q4_0 codes of one word (channel 2i in bits 4i.., channel 2i+1 in bits 16+4i..) times the fp16 scale
// in the low half of sc, as 8 fp16 in channel order: (w >> 4i) & 0x000F000F under the exponent pattern
// 0x6400 is the fp16 pair 1024 + code; subtracting 1032 gives code - 8 exactly, one packed multiply
// applies d (rounded once).
__device__ inline uint4 q4_dq8(uint32_t w, uint32_t sc) {
  const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)(sc & 0xFFFFu));
  const half2v_t d2 = {d, d};
  const half2v_t bias = {(_Float16)1032.0f, (_Float16)1032.0f};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = ((w >> (4 * i)) & 0x000F000Fu) | 0x64006400u;
    o[i] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(half2v_t, x) - bias) * d2);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// 8 INT8 codes (w0 then w1, lowest byte first) as 8 fp16 values, exactly: the biased byte under the
// exponent pattern 0x64 is 1024 + (c + 128), and subtracting 1152 leaves c.
__device__ inline uint4 i8_codes8(uint32_t w0, uint32_t w1) {
  const half2v_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t u = (j < 2 ? w0 : w1) ^ 0x80808080u;
    const uint32_t sel = (j & 1) ? 0x04030402u : 0x04010400u;
    o[j] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v_t, __builtin_amdgcn_perm(0x64646464u, u, sel)) - bias);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}
// 8 INT8 codes times the token's fp32 scale s, as 8 fp16 values fp16(fp32(s * code)).
__device__ inline uint4 i8_dq8(uint32_t w0, uint32_t w1, float s) {
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = (j < 2 ? w0 : w1) ^ 0x80808080u;
    const int b = 16 * (j & 1);
    const float a = (float)((w >> b) & 0xFFu) - 128.0f;  // exact
    const float c = (float)((w >> (b + 8)) & 0xFFu) - 128.0f;
    float as = a * s, cs = c * s;
    keep_fp32(as);  // rounded to fp32 first, then to fp16 (no fused mixed-precision product)
    keep_fp32(cs);
    const half2v_t hv = {(_Float16)as, (_Float16)cs};
    o[j] = __builtin_bit_cast(uint32_t, hv);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// 8 INT4 codes of one word (Q4_0's layout) less the token's zero point z, as 8 fp16 values, exactly:
// (w >> 4i) & 0x000F000F under the exponent pattern 0x6400 is the fp16 pair 1024 + code, and
// subtracting 1024 + z leaves code - z (|code - z| <= 15).
__device__ inline uint4 i4_codes8(uint32_t w, int z) {
  const _Float16 b = (_Float16)(float)(1024 + z);
  const half2v_t bias = {b, b};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = ((w >> (4 * i)) & 0x000F000Fu) | 0x64006400u;
    o[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v_t, x) - bias);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}
// 8 INT4 codes of one word as 8 fp16 values fp16(fp32(s * (code - z))).
__device__ inline uint4 i4_dq8(uint32_t w, float s, int z) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = (float)((int)((w >> (4 * i)) & 0xFu) - z) * s;
    float c = (float)((int)((w >> (16 + 4 * i)) & 0xFu) - z) * s;
    keep_fp32(a);  // rounded to fp32 first, then to fp16 (no fused mixed-precision product)
    keep_fp32(c);
    const half2v_t hv = {(_Float16)a, (_Float16)c};
    o[i] = __builtin_bit_cast(uint32_t, hv);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// The wave's 32 K code rows of 128 B (Q8_0, INT8: one byte per channel) into its LDS area, by buffer
// loads to LDS: load j brings rows 8j .. 8j+7 (1 KiB, contiguous in memory as in LDS), lane L's 16
// bytes to slot L % 8 of row 8j + L / 8.  Slot p of row r holds the row's chunk p ^ ((r / 2) % 8), so
// 16 lanes reading one chunk of 16 consecutive rows fall on 16 different 16-byte bank groups.
__device__ inline void k_rows128_to_lds(const unsigned char* kq, unsigned char* kbuf, int w, int lane) {
  const __amdgpu_buffer_rsrc_t kres =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(kq), (short)0, kQ8Codes, 0x00020000);
  const int rb = (32 * w + (lane >> 3)) * kDim;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kres, (__attribute__((address_space(3))) void*)(kbuf + j * 1024), 16,
                                             rb + 16 * ((lane & 7) ^ ((4 * j + (lane >> 4)) & 7)), j * 1024, 0,
                                             kNtLoad);
}
// Chunk c (16 bytes) of the wave's K code row r, as k_rows128_to_lds placed it.
__device__ inline uint4 k_row128_chunk(const unsigned char* kbuf, int r, int c) {
  return *reinterpret_cast<const uint4*>(kbuf + r * kDim + 16 * (c ^ ((r >> 1) & 7)));
}
// Wait until this wave's loads, but the `after` it issued last, have completed (vmcnt <= after, with
// expcnt and lgkmcnt left at their maxima), keeping the compiler from moving memory accesses across.
template <int after>
__device__ inline void wait_loads_but() {
  static_assert(after >= 0 && after < 16, "vmcnt's low field");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0F70 | after);
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// KV: the pools' KvType (fp16 tiles, Q8_0, Q4_0, or per-token INT8 or INT4 records).
template <int G, int KV = kKvFp16>
__device__ __forceinline__ void attn_tile(const Params& P, const uint16_t* __restrict__ q_h,
                                          const uint16_t* __restrict__ k_pool,
                                          const uint16_t* __restrict__ v_pool, int h, int phys, int ntok,
                                          float* __restrict__ part_o, float* __restrict__ part_ml,
                                          int n_parts, int part, unsigned char* smem,
                                          bool store = true, int tl_kind = -1) {
  const int tid = threadIdx.x & 255, w = tid >> 6, lane = tid & 63, lq = lane >> 4, lc = lane & 15;
  KVS_TL_BEGIN(P, tl_kind >= 0 ? tl_kind : P.tl_kind, 256)
  // Every load is issued up front, in the order the data is needed -- Q, K, then V -- and without
  // branches, so the compiler keeps them all in flight and waits only for what the next step needs.
  // Rows past ntok are still inside the tile: their K only feeds logits that are masked, their V is
  // zeroed after the load (a NaN tail times p = 0 would not be 0).
  half8_t qb[4];  // Q^T B operand: lane l holds head lc, 8 channels per MFMA m (below)
  uint4 kr[2][4], vr[8];
  uint4 vc[4];    // Q8_0 / Q4_0 / INT8: V codes and scales, dequantized when V is staged
  uint32_t vs[4];
  float ksc[2];    // INT8 / INT4: the fp32 scale of the lane's K token 32w + 16g + lc
  f32x4_t vsc;     // INT8 / INT4: the fp32 scales of the lane's 4 V tokens
  uint2 vq4[4];    // INT4: V codes of the lane's 4 tokens (16 channels each)
  uint32_t vz4 = 0;  // INT4: the zero points of the lane's 4 V tokens, one byte each
  if constexpr (KV == kKvFp16) {
    // fp16 tile: K rows of MFMA m are channels 32m + 8*lq .. +8
    const size_t off = ((size_t)phys * P.Hkv + h) * kTile;
    const uint16_t* Kt = k_pool + off;
    const uint16_t* Vt = v_pool + off;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint4 v = *reinterpret_cast<const uint4*>(q_h + (size_t)(lc < G ? lc : 0) * kDim + 32 * m + 8 * lq);
      qb[m] = __builtin_bit_cast(half8_t, lc < G ? v : make_uint4(0, 0, 0, 0));
    }
    // K goes straight into the wave's LDS rows (buffer loads to LDS): load j brings the wave's token
    // rows 4j .. 4j+3, 1 KiB contiguous in memory as in LDS, lane L's 16 bytes to LDS slot L % 16 of
    // row 4j + L / 16.  Slot p of row r holds the row's 16-byte chunk p ^ (r % 16), so the A-operand
    // reads below (16 rows, one chunk) fall on 16 different slots.  A load of 16 token rows x 64 B
    // in the A-operand layout straight from memory streams about 10% slower than these.
    {
      unsigned char* kbuf = smem + w * kWaveVBytes;
      const __amdgpu_buffer_rsrc_t kres =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Kt), (short)0, kTile * 2, 0x00020000);
      const int rb = (32 * w + (lane >> 4)) * (kDim * 2);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            kres, (__attribute__((address_space(3))) void*)(kbuf + j * 1024), 16,
            rb + 16 * ((lane & 15) ^ ((4 * j + (lane >> 4)) & 15)), j * 1024, 0, kNtLoad);
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 8; ++i) vr[i] = ld_stream16(Vt + (32 * w + 4 * i + lq) * kDim + 8 * lc);
    // The K rows are in LDS once every load of the wave but the 8 V loads issued after them has
    // completed.  The compiler does not order LDS reads after loads to LDS by itself.
    wait_loads_but<8>();
    {
      const unsigned char* kbuf = smem + w * kWaveVBytes;
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          kr[g][m] = *reinterpret_cast<const uint4*>(kbuf + (16 * g + lc) * (kDim * 2) + 16 * ((4 * m + lq) ^ lc));
    }
  } else if constexpr (KV == kKvQ4) {
    // Q4_0 record: as for Q8_0 below, a lane's K codes are the 32 channels 32*lq .. +32 of its
    // token (one block, one scale), here one 16-byte load, and MFMA m takes word m of them; V: lane l
    // takes one block (channels 32*(l%4) .. +32) of the wave's tokens l/4 and 16 + l/4.
    const size_t rec = ((size_t)phys * P.Hkv + h) * kQ4Record;
    const unsigned char* Kq = reinterpret_cast<const unsigned char*>(k_pool) + rec;
    const unsigned char* Vq = reinterpret_cast<const unsigned char*>(v_pool) + rec;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint4 v = *reinterpret_cast<const uint4*>(q_h + (size_t)(lc < G ? lc : 0) * kDim + 32 * lq + 8 * m);
      qb[m] = __builtin_bit_cast(half8_t, lc < G ? v : make_uint4(0, 0, 0, 0));
    }
    uint4 kc[2];
    uint32_t ks[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int tok = 32 * w + 16 * g + lc;
      kc[g] = ld_stream16(Kq + tok * (kDim / 2) + 16 * lq);
      ks[g] = *reinterpret_cast<const uint16_t*>(Kq + kQ4Codes + tok * 8 + 2 * lq);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int tok = 32 * w + 16 * i + (lane >> 2);
      vc[i] = ld_stream16(Vq + tok * (kDim / 2) + 16 * (lane & 3));
      vs[i] = *reinterpret_cast<const uint16_t*>(Vq + kQ4Codes + tok * 8 + 2 * (lane & 3));
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      kr[g][0] = q4_dq8(kc[g].x, ks[g]);
      kr[g][1] = q4_dq8(kc[g].y, ks[g]);
      kr[g][2] = q4_dq8(kc[g].z, ks[g]);
      kr[g][3] = q4_dq8(kc[g].w, ks[g]);
    }
  } else if constexpr (KV == kKvI4) {
    // INT4 record, one fp32 scale and one zero point per token: a lane's K codes are the 32 channels
    // 32*lq .. +32 of its token, as for Q4_0 (one 16-byte load, MFMA m takes word m); they enter the
    // product as the exact fp16 integers code - z, and the S rows are scaled by their tokens' fp32
    // scales afterwards, as for INT8.  V: lane l takes channels 16*(l%8) .. +16 (8 bytes of codes) of
    // the wave's four consecutive tokens 4*(l/8) .. +3, so their scales are one 16-byte load and their
    // zero points one 4-byte load; scaled when staged.
    const size_t rec = ((size_t)phys * P.Hkv + h) * kI4Record;
    const unsigned char* Kq = reinterpret_cast<const unsigned char*>(k_pool) + rec;
    const unsigned char* Vq = reinterpret_cast<const unsigned char*>(v_pool) + rec;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint4 v = *reinterpret_cast<const uint4*>(q_h + (size_t)(lc < G ? lc : 0) * kDim + 32 * lq + 8 * m);
      qb[m] = __builtin_bit_cast(half8_t, lc < G ? v : make_uint4(0, 0, 0, 0));
    }
    uint4 kc[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) kc[g] = ld_stream16(Kq + (32 * w + 16 * g + lc) * (kDim / 2) + 16 * lq);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = 32 * w + 4 * (lane >> 3) + i;
      vq4[i] = *reinterpret_cast<const uint2*>(Vq + tok * (kDim / 2) + 8 * (lane & 7));
    }
    // the scales and zero points last: they are needed after the codes
    int kz[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int tok = 32 * w + 16 * g + lc;
      ksc[g] = *reinterpret_cast<const float*>(Kq + kI4Scales + tok * 4);
      kz[g] = Kq[kI4Zeros + tok];
    }
    vsc = ld_stream16f(Vq + kI4Scales + (32 * w + 4 * (lane >> 3)) * 4);
    vz4 = *reinterpret_cast<const uint32_t*>(Vq + kI4Zeros + 32 * w + 4 * (lane >> 3));
    __builtin_amdgcn_sched_barrier(0);  // every load above is issued before the arithmetic below
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      kr[g][0] = i4_codes8(kc[g].x, kz[g]);
      kr[g][1] = i4_codes8(kc[g].y, kz[g]);
      kr[g][2] = i4_codes8(kc[g].z, kz[g]);
      kr[g][3] = i4_codes8(kc[g].w, kz[g]);
    }
  } else if constexpr (KV == kKvI8) {
    // INT8 record, one fp32 scale per token: K codes load as for Q8_0 below and enter the product
    // as exact fp16 integers; the product is scaled per token row afterwards, S = s_t * (code_t . q),
    // which keeps the scale in fp32 (a lane loads its own K token's scale; the S rows' scales come
    // from the lanes holding those tokens).  V: lane l takes channels 16*(l%8) .. +16 of the wave's four
    // consecutive tokens 4*(l/8) .. +3, so their scales are one 16-byte load; scaled when staged.
    const size_t rec = ((size_t)phys * P.Hkv + h) * kI8Record;
    const unsigned char* Kq = reinterpret_cast<const unsigned char*>(k_pool) + rec;
    const unsigned char* Vq = reinterpret_cast<const unsigned char*>(v_pool) + rec;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint4 v = *reinterpret_cast<const uint4*>(q_h + (size_t)(lc < G ? lc : 0) * kDim + 32 * lq + 8 * m);
      qb[m] = __builtin_bit_cast(half8_t, lc < G ? v : make_uint4(0, 0, 0, 0));
    }
    // K codes through LDS by whole rows (k_rows128_to_lds), then the V codes and the scales
    unsigned char* kbuf = smem + w * kWaveVBytes;
    k_rows128_to_lds(Kq, kbuf, w, lane);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = 32 * w + 4 * (lane >> 3) + i;
      vc[i] = ld_stream16(Vq + tok * kDim + 16 * (lane & 7));
    }
    // the scales last: they are needed after the codes (S scaling, V staging)
#pragma unroll
    for (int g = 0; g < 2; ++g) ksc[g] = *reinterpret_cast<const float*>(Kq + kQ8Codes + (32 * w + 16 * g + lc) * 4);
    vsc = ld_stream16f(Vq + kQ8Codes + (32 * w + 4 * (lane >> 3)) * 4);
    wait_loads_but<7>();  // the K rows have landed; 4 V code loads and 3 scale loads may not have
    uint4 kc[2][2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      kc[g][0] = k_row128_chunk(kbuf, 16 * g + lc, 2 * lq);
      kc[g][1] = k_row128_chunk(kbuf, 16 * g + lc, 2 * lq + 1);
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      kr[g][0] = i8_codes8(kc[g][0].x, kc[g][0].y);
      kr[g][1] = i8_codes8(kc[g][0].z, kc[g][0].w);
      kr[g][2] = i8_codes8(kc[g][1].x, kc[g][1].y);
      kr[g][3] = i8_codes8(kc[g][1].z, kc[g][1].w);
    }
  } else {
    // Q8_0 record (kv_type; llama.cpp's block format): a lane's K codes are the 32 channels
    // 32*lq .. +32 of its token -- one Q8_0 block, one scale -- and MFMA m takes channels
    // 32*lq + 8m .. +8 of them.  The k-slots of the product may be any permutation of the
    // channels as long as Q^T follows it, so Q^T is loaded in the same order.
    const size_t rec = ((size_t)phys * P.Hkv + h) * kQ8Record;
    const unsigned char* Kq = reinterpret_cast<const unsigned char*>(k_pool) + rec;
    const unsigned char* Vq = reinterpret_cast<const unsigned char*>(v_pool) + rec;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint4 v = *reinterpret_cast<const uint4*>(q_h + (size_t)(lc < G ? lc : 0) * kDim + 32 * lq + 8 * m);
      qb[m] = __builtin_bit_cast(half8_t, lc < G ? v : make_uint4(0, 0, 0, 0));
    }
    // K codes through LDS by whole rows (k_rows128_to_lds); the lane's K scales before them
    uint32_t ks[2];
#pragma unroll
    for (int g = 0; g < 2; ++g)
      ks[g] = *reinterpret_cast<const uint16_t*>(Kq + kQ8Codes + (32 * w + 16 * g + lc) * 8 + 2 * lq);
    unsigned char* kbuf = smem + w * kWaveVBytes;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
    k_rows128_to_lds(Kq, kbuf, w, lane);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
    // V: lane l takes channels 16*(l%8) .. +16 (half a Q8_0 block, one scale) of the wave's tokens
    // 8i + l/8, i < 4: 16-byte code loads, staged below as two 16-byte rows of fp16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = 32 * w + 8 * i + (lane >> 3);
      vc[i] = ld_stream16(Vq + tok * kDim + 16 * (lane & 7));
      vs[i] = *reinterpret_cast<const uint16_t*>(Vq + kQ8Codes + tok * 8 + 2 * ((lane & 7) >> 1));
    }
    wait_loads_but<8>();  // the K rows have landed; the 8 V loads may not have
    uint4 kc[2][2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      kc[g][0] = k_row128_chunk(kbuf, 16 * g + lc, 2 * lq);
      kc[g][1] = k_row128_chunk(kbuf, 16 * g + lc, 2 * lq + 1);
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      kr[g][0] = q8_dq8(kc[g][0].x, kc[g][0].y, ks[g]);
      kr[g][1] = q8_dq8(kc[g][0].z, kc[g][0].w, ks[g]);
      kr[g][2] = q8_dq8(kc[g][1].x, kc[g][1].y, ks[g]);
      kr[g][3] = q8_dq8(kc[g][1].z, kc[g][1].w, ks[g]);
    }
  }
  KVS_TL_MARK_LOADED(1)
  f32x4_t S[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    S[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 4; ++m)
      S[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, kr[g][m]), qb[m], S[g], 0, 0, 0);
  }
  // lane l holds S[token 32w + 16g + 4*lq + i][head lc]
  const float sl2 = P.scale_log2;
  float mx = -INFINITY;
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = 32 * w + 16 * g + 4 * lq + i;
      if constexpr (KV == kKvI8 || KV == kKvI4) S[g][i] *= __shfl(ksc[g], 4 * lq + i, 64);  // token 4lq + i's scale
      S[g][i] = tok < ntok ? S[g][i] * sl2 : -INFINITY;
      mx = fmaxf(mx, S[g][i]);
    }
  mx = fmaxf(mx, shfl_xor_f(mx, 16));
  mx = fmaxf(mx, shfl_xor_f(mx, 32));  // the wave's max for head lc (-inf if it has no tokens)
  half8_t pa;
  float ps = 0.f;
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = S[g][i] == -INFINITY ? 0.f : fast_exp2(S[g][i] - mx);
      const _Float16 ph = (_Float16)p;
      pa[4 * g + i] = ph;
      ps += (float)ph;
    }
  ps += shfl_xor_f(ps, 16);
  ps += shfl_xor_f(ps, 32);
  // V to LDS: chunk i holds the wave's tokens 4i..4i+3, one kVRow row each
  unsigned char* vbuf = smem + w * kWaveVBytes;
  if constexpr (KV == kKvQ4) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int t = 16 * i + (lane >> 2);  // the wave's token: chunk t / 4, row t % 4
      const bool in = 32 * w + t < ntok;
      unsigned char* row = vbuf + (t >> 2) * kVChunk + (t & 3) * kVRow + 64 * (lane & 3);
      const uint32_t cw[4] = {vc[i].x, vc[i].y, vc[i].z, vc[i].w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
        *reinterpret_cast<uint4*>(row + 16 * u) = in ? q4_dq8(cw[u], vs[i]) : make_uint4(0, 0, 0, 0);
    }
  } else if constexpr (KV == kKvQ8 || KV == kKvI8 || KV == kKvI4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // the wave's token: chunk t / 4, row t % 4
      const int t = KV == kKvQ8 ? 8 * i + (lane >> 3) : 4 * (lane >> 3) + i;
      const bool in = 32 * w + t < ntok;
      uint4 a, b;
      if constexpr (KV == kKvI4) {
        const int z = (int)((vz4 >> (8 * i)) & 0xFFu);
        a = i4_dq8(vq4[i].x, vsc[i], z);
        b = i4_dq8(vq4[i].y, vsc[i], z);
      } else if constexpr (KV == kKvI8) {
        a = i8_dq8(vc[i].x, vc[i].y, vsc[i]);
        b = i8_dq8(vc[i].z, vc[i].w, vsc[i]);
      } else {
        a = q8_dq8(vc[i].x, vc[i].y, vs[i]);
        b = q8_dq8(vc[i].z, vc[i].w, vs[i]);
      }
      unsigned char* row = vbuf + (t >> 2) * kVChunk + (t & 3) * kVRow + 32 * (lane & 7);
      *reinterpret_cast<uint4*>(row) = in ? a : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(row + 16) = in ? b : make_uint4(0, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool in = 32 * w + 4 * i + lq < ntok;
      *reinterpret_cast<uint4*>(vbuf + i * kVChunk + lq * kVRow + lc * 16) = in ? vr[i] : make_uint4(0, 0, 0, 0);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  f32x4_t O[8];
  // B operand of k-slots 8*lq + e: V[token 4*lq + e][16nn + lc] from chunk lq (e < 4) and
  // V[token 16 + 4*lq + e - 4][16nn + lc] from chunk 4 + lq (e >= 4)
  const unsigned char* vsrc = vbuf + lq * kVChunk + (lc >> 2) * kVRow + (lc & 3) * 8;
#pragma unroll
  for (int nn = 0; nn < 8; ++nn) {
    const v4s_t lo = lds_read_tr16(vsrc + nn * 32);
    const v4s_t hi = lds_read_tr16(vsrc + 4 * kVChunk + nn * 32);
    const half8_t vb = __builtin_bit_cast(half8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    O[nn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, vb, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  }
  __syncthreads();  // the V staging area becomes the fold buffer
  float* sm = reinterpret_cast<float*>(smem);  // [4 waves][16 heads]
  float* sl = sm + 64;                         // [4][16]
  float* so = sl + 64;                         // [4][G][128]
  if (lq == 0) { sm[w * 16 + lc] = mx; sl[w * 16 + lc] = ps; }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int head = 4 * lq + i;  // O rows are heads 4*lq + i
    if (head < G)
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) so[(w * G + head) * kDim + 16 * nn + lc] = O[nn][i];
  }
  __syncthreads();
  // one lane per (head, 4 channels); the (max, sum) pair goes with channel 0
  for (int idx = tid; store && idx < G * (kDim / 4); idx += 256) {
    const int j = idx / (kDim / 4), ch = (idx % (kDim / 4)) * 4;
    const float M = fmaxf(fmaxf(sm[j], sm[16 + j]), fmaxf(sm[32 + j], sm[48 + j]));
    float lsum = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float f = exp2_diff(sm[ww * 16 + j], M);
      const float* src = so + (ww * G + j) * kDim + ch;
      lsum += sl[ww * 16 + j] * f;
      acc.x += src[0] * f;
      acc.y += src[1] * f;
      acc.z += src[2] * f;
      acc.w += src[3] * f;
    }
    const size_t pr = (size_t)j * n_parts + part;
    *reinterpret_cast<float4*>(part_o + pr * kDim + ch) = acc;
    if (ch == 0) *reinterpret_cast<float2*>(part_ml + pr * 2) = make_float2(M, lsum);
  }
  KVS_TL_MARK(2)
}

constexpr int kMergeChunk = 1024;  // partials whose (max, sum) pairs sit in LDS at once
constexpr int kMergeFirst = 256;   // partials whose outputs are loaded before their count is known
constexpr int kMergeCh = 32;       // output channels one merge workgroup covers
constexpr int kMergeLdsFloats = 2 * kMergeChunk + 256 * 4 + 16;

// Log-sum-exp merge of channels [ch0, ch0 + kMergeCh) of one query head over its n (<= n_max)
// partials, by 256 lanes:
//   out = sum_s exp2(m_s - M) o_s / sum_s exp2(m_s - M) l_s,  M = max_s m_s.
// Lane t owns 4 channels (t % 8) of partial group t / 8 (32 groups).  The loads that do not depend on
// n -- the (max, sum) pairs of the first chunk and the first kMergeFirst partials' outputs -- are issued
// first, with clamped indices and no branches, so they travel with the loads that produce n.  Chunks
// of kMergeChunk partials keep a running (M, sum, accumulator) state; the 32 groups fold in LDS.
// n == 0 gives zeros.
__device__ inline void merge_head(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                  int n_max, int n, int ch0, float* __restrict__ out, float* lds) {
  constexpr int TPR = kMergeCh / 4;  // lanes per partial row
  constexpr int PG = 256 / TPR;      // partial groups
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  float* wts = lds;                  // [kMergeChunk]: max, then weight
  float* sums = wts + kMergeChunk;   // [kMergeChunk]
  float* fold = sums + kMergeChunk;  // [PG][kMergeCh]
  float* red = fold + 256 * 4;       // [8]
  const int c4 = ch0 + (tid % TPR) * 4, grp = tid / TPR;
  constexpr int R0 = kMergeChunk / 256, U0 = kMergeFirst / PG;
  float2 ml0[R0];
  const int m0 = min(n_max, kMergeChunk);
#pragma unroll
  for (int r = 0; r < R0; ++r) {
    const int s = tid + 256 * r;
    ml0[r] = *reinterpret_cast<const float2*>(part_ml + (size_t)min(s, m0 - 1) * 2);
  }
  float4 o0[U0];
  const int f0 = min(n_max, kMergeFirst);
#pragma unroll
  for (int u = 0; u < U0; ++u) {
    const int s = grp + PG * u;
    o0[u] = *reinterpret_cast<const float4*>(part_o + (size_t)min(s, f0 - 1) * kDim + c4);
  }
  float M = -INFINITY, Lsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto fma4 = [&](const float4& o, float f) {
    acc.x += o.x * f; acc.y += o.y * f; acc.z += o.z * f; acc.w += o.w * f;
  };
  for (int c0 = 0; c0 < n; c0 += kMergeChunk) {
    const int cn = min(kMergeChunk, n - c0);
    float cm = -INFINITY;
#pragma unroll
    for (int r = 0; r < R0; ++r) {
      const int s = tid + 256 * r;
      if (s < cn) {
        const float2 ml = c0 == 0 ? ml0[r] : *reinterpret_cast<const float2*>(part_ml + (size_t)(c0 + s) * 2);
        wts[s] = ml.x;
        sums[s] = ml.y;
        cm = fmaxf(cm, ml.x);
      }
    }
    cm = wave_max_f32(cm);
    if (lane == 0) red[w] = cm;
    __syncthreads();
    const float Mn = fmaxf(M, fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
    const float resc = exp2_diff(M, Mn);  // 0 while nothing has been accumulated
    M = Mn;
    float cl = 0.f;
#pragma unroll
    for (int r = 0; r < R0; ++r) {  // each lane rewrites only the entries it wrote
      const int s = tid + 256 * r;
      if (s < cn) {
        const float f = exp2_diff(wts[s], M);
        wts[s] = f;
        cl += sums[s] * f;
      }
    }
    cl = wave_sum_f32(cl);
    if (lane == 0) red[4 + w] = cl;
    __syncthreads();  // weights and chunk sums visible
    acc.x *= resc; acc.y *= resc; acc.z *= resc; acc.w *= resc;
    int s_from = 0;
    if (c0 == 0) {
#pragma unroll
      for (int u = 0; u < U0; ++u) {
        const int s = grp + PG * u;
        if (s < cn) fma4(o0[u], wts[s]);
      }
      s_from = kMergeFirst;
    }
    for (int s0 = s_from + grp; s0 < cn; s0 += 8 * PG) {  // the rest, 8 loads in flight
      float4 o[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int s = min(s0 + PG * u, cn - 1);
        o[u] = *reinterpret_cast<const float4*>(part_o + (size_t)(c0 + s) * kDim + c4);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int s = s0 + PG * u;
        if (s < cn) fma4(o[u], wts[s]);
      }
    }
    Lsum = Lsum * resc + red[4] + red[5] + red[6] + red[7];
    __syncthreads();  // red[] and wts[] are rewritten by the next chunk
  }
  *reinterpret_cast<float4*>(fold + grp * kMergeCh + (c4 - ch0)) = acc;
  __syncthreads();
  if (tid < kMergeCh) {
    float a = 0.f;
#pragma unroll 8
    for (int g = 0; g < PG; ++g) a += fold[g * kMergeCh + tid];
    out[ch0 + tid] = Lsum > 0.f ? a / Lsum : 0.f;
  }
}

// Merge of channels [ch0, ch0 + 16) of one query head over its n (<= n_max) partials by ONE wave: no
// workgroup barriers, the reductions go through DPP and the wave's own LDS.  Lane l owns channels
// ch0 + 4(l % 4) .. +3 of partials l / 4 + 16u; the outputs of the first 16 * kMergeWaveRows partials
// and the (max, sum) pairs of the first 64 * kMergeWaveMl are requested together, with indices clamped
// to n_max rather than n, so that they travel with the loads that produce n (entries past n are read
// and not used).  wl: this wave's LDS scratch of >= n + 256 floats.  n == 0 gives zeros.
constexpr int kMergeChWave = 16;
constexpr int kMergeWaveRows = 12;
constexpr int kMergeWaveMl = 3;
// n_of() gives n; it is called after those requests, so that its own loads' waits (and branches) come
// after them.
template <typename NFn>
__device__ inline void merge_head_wave(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                       int n_max, NFn n_of, int ch0, float* __restrict__ out, float* wl,
                                       unsigned long long* tl_rec = nullptr) {
  const int lane = threadIdx.x & 63, cg = lane & 3, pg = lane >> 2;
  auto ld_ml = [&](int s) { return *reinterpret_cast<const float2*>(part_ml + (size_t)s * 2); };
  auto ld_o = [&](int s) { return *reinterpret_cast<const float4*>(part_o + (size_t)s * kDim + ch0 + 4 * cg); };
  const int last = max(n_max - 1, 0);
  float2 ml[kMergeWaveMl];
#pragma unroll
  for (int r = 0; r < kMergeWaveMl; ++r) ml[r] = ld_ml(min(lane + 64 * r, last));
  float4 o[kMergeWaveRows];
#pragma unroll
  for (int u = 0; u < kMergeWaveRows; ++u) o[u] = ld_o(min(pg + 16 * u, last));
  const int n = n_of();
#ifdef KVS_TIMELINE
  if (tl_rec) {  // the timeline build: the loads above have landed
    wait_mem();
    tl_rec[1] = __builtin_amdgcn_s_memrealtime();
  }
#endif
  // The preloaded slots are folded without branches: a slot past n (its load clamped, its value
  // anything, NaN included) is selected away, so the LDS reads below are issued together instead of
  // one round trip per branch.
  float M = -INFINITY;
#pragma unroll
  for (int r = 0; r < kMergeWaveMl; ++r) M = fmaxf(M, lane + 64 * r < n ? ml[r].x : -INFINITY);
  for (int s = lane + 64 * kMergeWaveMl; s < n; s += 64) M = fmaxf(M, ld_ml(s).x);
  M = wave_max_f32(M);
  float L = 0.f;
  auto weigh = [&](int s, float2 m) {
    const float w = exp2_diff(m.x, M);
    wl[s] = w;
    L += m.y * w;
  };
#pragma unroll
  for (int r = 0; r < kMergeWaveMl; ++r) {
    const int s = lane + 64 * r;
    const bool ok = s < n;
    const float w = exp2_diff(ml[r].x, M);
    if (ok) wl[s] = w;
    L += ok ? ml[r].y * w : 0.f;
  }
  for (int s = lane + 64 * kMergeWaveMl; s < n; s += 64) weigh(s, ld_ml(s));
  L = wave_sum_f32(L);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto fma4 = [&](const float4& v, float f) {
    acc.x += v.x * f; acc.y += v.y * f; acc.z += v.z * f; acc.w += v.w * f;
  };
  float wu[kMergeWaveRows];  // slots past n read LDS inside the wave's area (it holds n_max + 256)
#pragma unroll
  for (int u = 0; u < kMergeWaveRows; ++u) wu[u] = wl[pg + 16 * u];
#pragma unroll
  for (int u = 0; u < kMergeWaveRows; ++u) {
    const bool ok = pg + 16 * u < n;
    acc.x += ok ? o[u].x * wu[u] : 0.f;
    acc.y += ok ? o[u].y * wu[u] : 0.f;
    acc.z += ok ? o[u].z * wu[u] : 0.f;
    acc.w += ok ? o[u].w * wu[u] : 0.f;
  }
  for (int s = pg + 16 * kMergeWaveRows; s < n; s += 64) {  // the rest, 4 loads in flight
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = ld_o(min(s + 16 * u, n - 1));
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (s + 16 * u < n) fma4(v[u], wl[s + 16 * u]);
  }
  float* red = wl + n;  // [16 partial groups][16 channels]
  *reinterpret_cast<float4*>(red + pg * kMergeChWave + 4 * cg) = acc;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < kMergeChWave) {
    float r[16];  // every read issued before the sums
#pragma unroll
    for (int g = 0; g < 16; ++g) r[g] = red[g * kMergeChWave + lane];
#pragma unroll
    for (int step = 1; step < 16; step *= 2)
#pragma unroll
      for (int g = 0; g < 16; g += 2 * step) r[g] += r[g + step];
    out[ch0 + lane] = L > 0.f ? r[0] / L : 0.f;
  }
}

// Writes an empty partial (max -inf, sum 0, zero output) for the g query heads of a tile that names
// no valid block.
template <int G>
__device__ inline void empty_partial(float* part_o, float* part_ml, int n_parts, int part) {
  for (int idx = threadIdx.x; idx < G * kDim; idx += blockDim.x) {
    const int j = idx / kDim, c = idx % kDim;
    part_o[((size_t)j * n_parts + part) * kDim + c] = 0.f;
    if (c == 0) *reinterpret_cast<float2*>(part_ml + ((size_t)j * n_parts + part) * 2) = make_float2(-INFINITY, 0.f);
  }
}

// One attention work item of KV head h of sequence seq.  With IL, x < n_il_max names the x-th
// Initial/Local tile; otherwise (or beyond n_il_max with IL) x names selected tile i = x - (IL ?
// n_il_max : 0), a logical block id in A.sel, or a physical one when PHYS.  Items past the
// sequence's own counts do nothing; table entries or selections outside the table give an empty
// partial instead of a read outside the pools' rows.
template <int G, bool IL, bool PHYS, int KV = kKvFp16>
__device__ __forceinline__ void attn_item(const AttnArgs& A, int x, int h, int seq, unsigned char* smem,
                                          int tl_kind = -1) {
  const Params& P = A.P;
  const bool is_il = IL && x < A.n_il_max;
  const int i = IL ? x - A.n_il_max : x;  // selected index when !is_il
  const size_t grow = (size_t)seq * P.G + (P.mode == kSeparate ? h : 0);
  // the loads that do not depend on the length first
  const int L = A.seq_lens[seq];
  int cnt = 0, v = -1;
  if (P.topk > 0) {
    cnt = A.sel_count[grow];
    v = A.sel[grow * P.topk + (is_il ? 0 : i)];
  }
  const TileList tl = tiles_of(L, P, 0);
  const int n_il = tl.nI + tl.nLoc;
  const int32_t* trow = A.table + (size_t)seq * A.max_blocks;
  int phys, ntok, part;
  if (is_il) {
    if (x >= n_il) return;
    const int2 t = il_tile(tl, x);
    phys = t.x < A.max_blocks ? trow[t.x] : -1;
    ntok = t.y;
    part = x;
  } else {
    if (i >= tiles_of(L, P, cnt).k) return;
    if (PHYS) phys = v;
    else phys = v >= 0 && v < A.max_blocks ? trow[v] : -1;
    ntok = kBlock;
    part = n_il + i;
  }
  const size_t head0 = (size_t)seq * P.Hq + (size_t)h * G;
  float* po = A.part_o + head0 * A.max_parts * kDim;
  float* pml = A.part_ml + head0 * A.max_parts * 2;
  if (phys < 0) {
    empty_partial<G>(po, pml, A.max_parts, part);
    return;
  }
  attn_tile<G, KV>(P, A.q + head0 * kDim, A.k_pool, A.v_pool, h, phys, ntok, po, pml, A.max_parts, part, smem,
                   true, tl_kind);
}

// Merge of channels [16c, 16c + 16) of query head j of sequence seq by one wave (merge_head_wave).
// The sequence's length and the group's selection count are loaded first, without branches (the
// count through a buffer load that reads 0 when there is no selection), so that they travel with the
// partials' loads.
__device__ inline void merge_item_wave(const AttnArgs& A, int j, int c, int seq, float* wl,
                                       unsigned long long* tl_rec = nullptr) {
  const Params& P = A.P;
  const int L = A.seq_lens[seq];
  const __amdgpu_buffer_rsrc_t rc =
      span_rsrc(A.sel_count + (size_t)seq * P.G + (P.mode == kSeparate ? j / P.g : 0), P.topk > 0 ? 4 : 0);
  const int cnt = (int)__builtin_amdgcn_raw_buffer_load_b32(rc, 0, 0, 0);
  const size_t hp = (size_t)seq * P.Hq + j;
  merge_head_wave(A.part_o + hp * A.max_parts * kDim, A.part_ml + hp * A.max_parts * 2, A.max_parts,
                  [&]() {
                    const TileList tl = tiles_of(L, P, cnt);
                    return tl.nI + tl.nLoc + tl.k;
                  },
                  c * kMergeChWave, A.out + hp * kDim, wl, tl_rec);
}

// Merge of channel quarter q4 of query head j of sequence seq over its n_il + k partials into out.
__device__ inline void merge_item(const AttnArgs& A, int j, int q4, int seq, float* lds) {
  const Params& P = A.P;
  const int L = A.seq_lens[seq];
  const int cnt = P.topk > 0 ? A.sel_count[(size_t)seq * P.G + (P.mode == kSeparate ? j / P.g : 0)] : 0;
  const TileList tl = tiles_of(L, P, cnt);
  const int n = tl.nI + tl.nLoc + tl.k;
  const size_t hp = (size_t)seq * P.Hq + j;
  merge_head(A.part_o + hp * A.max_parts * kDim, A.part_ml + hp * A.max_parts * 2, A.max_parts, n,
             q4 * kMergeCh, A.out + hp * kDim, lds);
}

}  // namespace kvs
