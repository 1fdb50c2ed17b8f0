// Exact attention over a list of K/V tiles on the matrix cores, for one workgroup of 256 lanes
// (used by kvs_sparse_decode_attn and kvs_decode_step).
// KTransformers long-context sparse attention (lmnt.cn): §4.2 Initial and Local are always attended
// with the selected Context blocks in between; §4.6 attn(query, kvcache_after_retrieval) with logits
// scaled by 1/sqrt(head_dim).
//
// One call covers a contiguous range of the attended tiles of one (sequence, KV head) and all g <= 16
// query heads reading that head, padded to the 16 rows of v_mfma_f32_16x16x32_f16.  Each of the 4
// waves owns 32 token rows of a tile:
//   S = K Q^T: K rows come straight from HBM in the A-operand layout (lane l: token l%16, channels
//     8*(l/16)..+8 of a 32-channel chunk: each load is 16 tokens x 64 contiguous bytes); Q^T is a
//     register-resident B operand.
//   online softmax in the exp2 domain per head (the 4 lanes holding one head combine with two
//     shuffles); P is rounded to fp16 and the row sums use the rounded values.
//   O += P V: P is already in the A-operand layout (k-slot 8*(l/16)+e holds token 16*(e/4)+4*(l/16)+e%4),
//     V passes through LDS in rows of 4 tokens padded to 1056 B so the transposed 16-bit reads of the B
//     operand are free of bank conflicts.
// The 4 waves fold through LDS into one partial (max, sum, unnormalised output) per head.
#pragma once

#include "kvs_device.h"

namespace kvs {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaveVBytes = 8 * 1056;                // V staging per wave
constexpr int kMaxItemTiles = 32;                     // tiles one call may cover
constexpr int kTileListOff = 4 * kWaveVBytes;         // LDS copy of the call's tile list
constexpr int kAttnLdsBytes = kTileListOff + kMaxItemTiles * 8;  // also >= fold buffers for G <= 16

// Issue the loads of one tile: K in the A-operand layout, V rows coalesced (4 rows per wave load).
__device__ inline void load_tile(const uint16_t* __restrict__ Kt, const uint16_t* __restrict__ Vt,
                                 int ntok, int w, int lq, int lc, uint4 (&kr)[2][4], uint4 (&vr)[8]) {
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int tok = 32 * w + 16 * g + lc;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      kr[g][m] = tok < ntok ? ld_stream16(Kt + tok * kDim + 32 * m + 8 * lq) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int tok = 32 * w + 4 * i + lq;
    vr[i] = tok < ntok ? ld_stream16(Vt + tok * kDim + 8 * lc) : make_uint4(0, 0, 0, 0);
  }
}

// Partial of heads h*G .. h*G+G-1 over tiles [0, n) given by tile(i) -> {physical id, tokens}
// (n <= kMaxItemTiles).  Writes part_o[j * n_parts + part][128] and
// part_ml[(j * n_parts + part) * 2 + {0: max, 1: sum}] for j < G (arrays already offset to the first
// query head of h).  n == 0 writes max = -inf only.  The next tile's K and V are loaded while the
// current one is computed.  COH: the partials are read by another workgroup of the same kernel.
template <int G, bool COH, typename TileFn>
__device__ __forceinline__ void attn_partial(const Params& P, const uint16_t* __restrict__ q_h,
                                    const uint16_t* __restrict__ k_pool,
                                    const uint16_t* __restrict__ v_pool, int h, int n, TileFn tile,
                                    float* __restrict__ part_o, float* __restrict__ part_ml,
                                    int n_parts, int part, unsigned char* smem) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lq = lane >> 4, lc = lane & 15;
  if (n <= 0) {
    if (tid < G) {
      float* dst = part_ml + ((size_t)tid * n_parts + part) * 2;
      if constexpr (COH) st_coh(dst, -INFINITY); else *dst = -INFINITY;
    }
    return;
  }
  unsigned char* vbuf = smem + w * kWaveVBytes;
  int2* ltiles = reinterpret_cast<int2*>(smem + kTileListOff);
  if (tid < n) ltiles[tid] = tile(tid);

  half8_t qb[4];  // Q^T B operand: lane l holds head lc, channels 32m + 8*lq .. +8
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (lc < G) v = *reinterpret_cast<const uint4*>(q_h + (size_t)lc * kDim + 32 * m + 8 * lq);
    qb[m] = __builtin_bit_cast(half8_t, v);
  }
  const float sl2 = P.scale_log2;
  float m_run = -INFINITY, l_run = 0.f;  // softmax state of head lc (identical in its 4 lanes)
  f32x4_t O[8];
#pragma unroll
  for (int nn = 0; nn < 8; ++nn) O[nn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  __syncthreads();  // tile list visible

  uint4 kr[2][4], vr[8];
  int2 tv = ltiles[0];
  {
    const size_t off = ((size_t)tv.x * P.Hkv + h) * kTile;
    load_tile(k_pool + off, v_pool + off, tv.y, w, lq, lc, kr, vr);
  }
  for (int ti = 0; ti < n; ++ti) {
    const int ntok = tv.y;
    // stage this tile's V: chunk i holds the wave's tokens 4i..4i+3, row stride 256 B
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<uint4*>(vbuf + i * 1056 + lq * 256 + lc * 16) = vr[i];
    f32x4_t S[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      S[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 4; ++m)
        S[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, kr[g][m]), qb[m], S[g], 0, 0, 0);
    }
    // prefetch the next tile into the now free registers
    if (ti + 1 < n) {
      tv = ltiles[ti + 1];
      const size_t off = ((size_t)tv.x * P.Hkv + h) * kTile;
      load_tile(k_pool + off, v_pool + off, tv.y, w, lq, lc, kr, vr);
    }
    // lane l holds S[token 32w + 16g + 4*lq + i][head lc]
    float mx = -INFINITY;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 32 * w + 16 * g + 4 * lq + i;
        S[g][i] = tok < ntok ? S[g][i] * sl2 : -INFINITY;
        mx = fmaxf(mx, S[g][i]);
      }
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const float mn = fmaxf(m_run, mx);
    const float alpha = exp2_diff(m_run, mn);
    m_run = mn;
    half8_t pa;
    float ps = 0.f;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = S[g][i] == -INFINITY ? 0.f : fast_exp2(S[g][i] - mn);
        const _Float16 ph = (_Float16)p;
        pa[4 * g + i] = ph;
        ps += (float)ph;
      }
    l_run = l_run * alpha + ps;
    // O rows are heads 4*lq + i: fetch those heads' rescale factors from lanes 4*lq + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ai = __shfl(alpha, 4 * lq + i, 64);
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) O[nn][i] *= ai;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const _Float16* vh = reinterpret_cast<const _Float16*>(vbuf);
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) {
      half8_t vb;  // B operand: V[token of k-slot 8*lq + e][channel 16nn + lc]
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int chunk = e < 4 ? lq : 4 + lq;
        vb[e] = vh[(chunk * 1056 + (e & 3) * 256) / 2 + 16 * nn + lc];
      }
      O[nn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, vb, O[nn], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  l_run += shfl_xor_f(l_run, 16);
  l_run += shfl_xor_f(l_run, 32);
  __syncthreads();  // the V staging area becomes the fold buffer
  float* sm = reinterpret_cast<float*>(smem);  // [4 waves][16 heads]
  float* sl = sm + 64;                         // [4][16]
  float* so = sl + 64;                         // [4][G][128]
  if (lq == 0) { sm[w * 16 + lc] = m_run; sl[w * 16 + lc] = l_run; }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int head = 4 * lq + i;
    if (head < G)
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) so[(w * G + head) * kDim + 16 * nn + lc] = O[nn][i];
  }
  __syncthreads();
  // one lane per (head, 4 channels); the (max, sum) pair goes with channel 0
  const __amdgpu_buffer_rsrc_t ro = coh_rsrc(part_o), rml = coh_rsrc(part_ml);
  for (int idx = tid; idx < G * (kDim / 4); idx += 256) {
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
    if constexpr (COH) {
      st_coh_f4(ro, (int)((pr * kDim + ch) * 4), acc);
      if (ch == 0) st_coh_f2(rml, (int)(pr * 8), make_float2(M, lsum));
    } else {
      *reinterpret_cast<float4*>(part_o + pr * kDim + ch) = acc;
      if (ch == 0) *reinterpret_cast<float2*>(part_ml + pr * 2) = make_float2(M, lsum);
    }
  }
  __syncthreads();  // smem is reused by the caller's next item
}

constexpr int kMaxParts = 256;  // partials one merge combines (plans keep n_parts <= this)
// LDS floats merge_heads needs: weights and sums [16][kMaxParts], totals [16], reduction [4][16*64*2].
constexpr int kMergeLdsFloats = 2 * 16 * kMaxParts + 16 + 4 * 16 * 64 * 2 / 4;

// Log-sum-exp merge of n_used (<= kMaxParts) partials for each of G query heads into out[j][128],
// by 256 lanes.  Parts whose max is -inf are empty.  Round 1 loads every (max, sum) pair in parallel
// and turns them into per-head weights in LDS; round 2 has each lane accumulate one or more
// (head, channel pair) columns over its share of the parts with independent 8-byte loads.
// COH: the partials were written by other workgroups of the same kernel.
template <int G, bool COH>
__device__ __forceinline__ void merge_heads(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                   int n_parts, int n_used, float* __restrict__ out, float* lds) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  constexpr int TPC = G >= 4 ? 1 : 4 / G;  // lanes per (head, channel pair) column
  constexpr int CPT = G >= 4 ? G / 4 : 1;  // columns per lane
  float* wts = lds;                        // [G][kMaxParts]: max, then weight
  float* sums = wts + 16 * kMaxParts;      // [G][kMaxParts]
  float* tot = sums + 16 * kMaxParts;      // [G]
  float2* red = reinterpret_cast<float2*>(tot + 16);  // [TPC][G * 64]
  const __amdgpu_buffer_rsrc_t ro = coh_rsrc(part_o), rml = coh_rsrc(part_ml);
  auto ld2 = [&](const float* p, bool is_ml) -> float2 {
    if constexpr (COH) {
      const float* base = is_ml ? part_ml : part_o;
      return ld_coh_f2(is_ml ? rml : ro, (int)((p - base) * 4));
    } else {
      return *reinterpret_cast<const float2*>(p);
    }
  };
  for (int idx = tid; idx < G * n_used; idx += 256) {
    const int j = idx / n_used, s = idx % n_used;
    const float2 ml = ld2(part_ml + ((size_t)j * n_parts + s) * 2, true);
    wts[j * kMaxParts + s] = ml.x;
    sums[j * kMaxParts + s] = ml.y;
  }
  __syncthreads();
  for (int j = w; j < G; j += 4) {
    float M = -INFINITY;
    for (int s = lane; s < n_used; s += 64) M = fmaxf(M, wts[j * kMaxParts + s]);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) M = fmaxf(M, shfl_xor_f(M, m));
    float L = 0.f;
    for (int s = lane; s < n_used; s += 64) {
      const float f = exp2_diff(wts[j * kMaxParts + s], M);
      wts[j * kMaxParts + s] = f;
      L += sums[j * kMaxParts + s] * f;
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) L += shfl_xor_f(L, m);
    if (lane == 0) tot[j] = L;
  }
  __syncthreads();
  const int sub = tid % TPC;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int col = tid / TPC + c * (256 / TPC);  // column = head * 64 + channel pair
    const int j = col / 64, pcol = col % 64;
    const float* po = part_o + (size_t)j * n_parts * kDim + 2 * pcol;
    float a0 = 0.f, a1 = 0.f;
    for (int s0 = sub; s0 < n_used; s0 += 8 * TPC) {  // 8 independent loads in flight
      float2 o[8];
      float f[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int s = s0 + u * TPC;
        const bool ok = s < n_used;
        f[u] = ok ? wts[j * kMaxParts + s] : 0.f;
        o[u] = ld2(po + (size_t)(ok ? s : 0) * kDim, false);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {  // an empty part's output is never used
        a0 += f[u] != 0.f ? o[u].x * f[u] : 0.f;
        a1 += f[u] != 0.f ? o[u].y * f[u] : 0.f;
      }
    }
    if constexpr (TPC == 1) {
      const float L = tot[j];
      const float inv = L > 0.f ? 1.f / L : 0.f;
      *reinterpret_cast<float2*>(out + (size_t)j * kDim + 2 * pcol) = make_float2(a0 * inv, a1 * inv);
    } else {
      red[sub * (G * 64) + col] = make_float2(a0, a1);
    }
  }
  if constexpr (TPC > 1) {
    __syncthreads();
    for (int col = tid; col < G * 64; col += 256) {
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int r = 0; r < TPC; ++r) { a0 += red[r * (G * 64) + col].x; a1 += red[r * (G * 64) + col].y; }
      const int j = col / 64, pcol = col % 64;
      const float L = tot[j];
      const float inv = L > 0.f ? 1.f / L : 0.f;
      *reinterpret_cast<float2*>(out + (size_t)j * kDim + 2 * pcol) = make_float2(a0 * inv, a1 * inv);
    }
  }
  __syncthreads();
}

}  // namespace kvs
