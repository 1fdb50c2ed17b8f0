// Dynamic reps: every cached token's cumulative attention score, and each block's top tokens as its
// reps.  The KTransformers long-context article (§4.3, rep table) names the method -- each token's
// accumulated attention score, the highest-scoring tokens of a block become its reps -- and leaves
// the scoring method open.  Here a token's score is the attention it receives from the n_obs
// observation queries (the last n_obs tokens of the cache, each attending causally, scale
// 1/sqrt(d)), summed over those queries and the query heads of the selection group.
//
// The probabilities need each query row's softmax normaliser over all of its keys, so the scores
// take three passes over K (the fourth only for SHARED):
//  1. imp_stats_kernel, one workgroup per (block, KV head, sequence): the K tile in the A-operand
//     layout straight from HBM and the rows' queries staged in LDS are requested together; then
//     S = K Q^T on the matrix cores for every row (observation query, query head of the KV head),
//     16 rows at a time, and each wave keeps its 32 tokens' max and sum of exp2 per row -- a
//     partial per (row, wave), so no barrier orders the waves.
//  2. imp_merge_kernel, one workgroup per (sequence, KV head, row): log-sum-exp of the row's partials.
//  3. imp_accum_kernel, one workgroup per (block, KV head, sequence): the same products again,
//     p = exp2(z - M) / l summed over the 16 rows of a DPP row and over row groups in registers;
//     SEPARATE stores the score row of the KV head, SHARED a per-head row that
//  4. imp_sum_kernel adds over the KV heads.
// dyn_reps_kernel: one wave per (block, KV head, sequence) ranks the block's 128 scores by counting
// (higher score, or equal and lower token, beats) and copies the K rows of the rep_num best, in
// ascending token order, into the rep pool; a Dynamic block is then scored like Fix.
// Over a quantized cache the products take the codes as exact fp16 integers and are scaled in fp32
// (per 32-channel block, or per token for INT8), and the reps are the chosen rows' cached values
// rounded to fp16, as the other reps of such a cache.
#include "attn_core.h"
#include "kvs_launch.h"
#include "quant_rows.h"

namespace kvs {

namespace {

// K tile of (phys, h) in the A-operand layout of attn_tile: lane (lc, lq) of wave w, token group g
// (16 tokens), MFMA m: token 32w + 16g + lc, channels 32m + 8lq .. +8 -- so MFMA m spans channels
// 32m .. 32m + 31, one quantization block.  A quantized record gives its codes as exact fp16 integers
// (Q4_0: code - 8) and the scales of the lane's S rows (tokens 32w + 16g + 4lq + i): Q8_0 / Q4_0 the
// fp16 scales [4 tokens][4 blocks] (32 bytes), INT8 the 4 tokens' fp32 scales (sc[g][0]).  The
// products are scaled in fp32 (imp_s), so the logits see the cached values without an fp16 rounding.
template <int KV>
struct KTile {
  uint4 kr[2][4];
  uint4 sc[2][2];
};

template <int KV>
__device__ inline void load_k_tile(const void* __restrict__ k_pool, size_t tile, KTile<KV>& T) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lq = lane >> 4, lc = lane & 15;
  if constexpr (KV == kKvFp16) {
    const uint16_t* Kt = static_cast<const uint16_t*>(k_pool) + tile * kTile;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int m = 0; m < 4; ++m) T.kr[g][m] = ld_stream16(Kt + (32 * w + 16 * g + lc) * kDim + 32 * m + 8 * lq);
  } else {
    constexpr int kRec = KV == kKvQ4 ? kQ4Record : KV == kKvI8 ? kI8Record : KV == kKvI4 ? kI4Record : kQ8Record;
    constexpr int kCodes = KV == kKvQ4 || KV == kKvI4 ? kQ4Codes : kQ8Codes;  // INT4: the scales follow
    const unsigned char* rec = static_cast<const unsigned char*>(k_pool) + tile * (size_t)kRec;
    uint2 raw[2][4];  // every load first, then the conversions
    int kz[2] = {0, 0};  // INT4: the zero point of the lane's K token
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int tok = 32 * w + 16 * g + lc;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if constexpr (KV == kKvQ4 || KV == kKvI4)
          raw[g][m].x = *reinterpret_cast<const uint32_t*>(rec + tok * (kDim / 2) + 4 * (4 * m + lq));
        else
          raw[g][m] = *reinterpret_cast<const uint2*>(rec + tok * kDim + 32 * m + 8 * lq);
      }
      const int t0 = 32 * w + 16 * g + 4 * lq;
      if constexpr (KV == kKvI8 || KV == kKvI4) {
        T.sc[g][0] = *reinterpret_cast<const uint4*>(rec + kCodes + t0 * 4);
        if constexpr (KV == kKvI4) kz[g] = rec[kI4Zeros + tok];
      } else {
        T.sc[g][0] = *reinterpret_cast<const uint4*>(rec + kCodes + t0 * 8);
        T.sc[g][1] = *reinterpret_cast<const uint4*>(rec + kCodes + t0 * 8 + 16);
      }
    }
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        T.kr[g][m] = KV == kKvQ4   ? q4_dq8(raw[g][m].x, 0x3C00u)  // fp16 1.0: code - 8 exactly
                     : KV == kKvI4 ? i4_codes8(raw[g][m].x, kz[g])   // code - z exactly
                                   : i8_codes8(raw[g][m].x, raw[g][m].y);
  }
}

constexpr int kImpRows = 128;  // rows (observation query, query head) staged in LDS at a time

// Rows [r0, r0 + kImpRows) of KV head h into LDS, 256 B each: row r = observation r >> gsh, query head
// (h << gsh) + (r & (g - 1)) (g = 2^gsh query heads per KV head).  Rows past n_rows are zero.  All 8
// loads of a lane are issued, with clamped rows and no branch, before the first LDS store.
__device__ inline void stage_q_rows(const uint16_t* __restrict__ q_seq, int h, int gsh, int Hq, int n_rows,
                                    int r0, uint4* qs) {
  constexpr int U = kImpRows * 16 / 256;
  uint4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int x = threadIdx.x + 256 * u, r = r0 + x / 16, c = x % 16;
    const int rr = r < n_rows ? r : 0;
    v[u] = *reinterpret_cast<const uint4*>(
        q_seq + ((size_t)(rr >> gsh) * Hq + (h << gsh) + (rr & ((1 << gsh) - 1))) * kDim + 8 * c);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int x = threadIdx.x + 256 * u;
    qs[x] = r0 + x / 16 < n_rows ? v[u] : make_uint4(0, 0, 0, 0);
  }
}

// Q^T B operand of staged rows rg*16 .. +16: lane (lc, lq) holds row lc, channels 32m + 8lq .. +8.
__device__ inline void q_rows_from_lds(const uint4* qs, int rg, half8_t (&qb)[4]) {
  const int lane = threadIdx.x & 63, lq = lane >> 4, lc = lane & 15;
#pragma unroll
  for (int m = 0; m < 4; ++m) qb[m] = __builtin_bit_cast(half8_t, qs[(rg * 16 + lc) * 16 + 4 * m + lq]);
}

// S = K Q^T for token group gg of this wave and the 16 rows of qb (lane: tokens 4lq + i, row lc).
// Q8_0 / Q4_0: each block's product is scaled by its token's block scale before the sum over blocks;
// INT8 / INT4: the sum is scaled by the token's scale.
template <int KV>
__device__ inline f32x4_t imp_s(const KTile<KV>& T, const half8_t (&qb)[4], int gg) {
  f32x4_t S = {0.f, 0.f, 0.f, 0.f};
  if constexpr (KV == kKvFp16 || KV == kKvI8 || KV == kKvI4) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
      S = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, T.kr[gg][m]), qb[m], S, 0, 0, 0);
    if constexpr (KV == kKvI8 || KV == kKvI4) {
      const f32x4_t s = __builtin_bit_cast(f32x4_t, T.sc[gg][0]);
#pragma unroll
      for (int i = 0; i < 4; ++i) S[i] *= s[i];
    }
  } else {
    const uint32_t sw[8] = {T.sc[gg][0].x, T.sc[gg][0].y, T.sc[gg][0].z, T.sc[gg][0].w,
                            T.sc[gg][1].x, T.sc[gg][1].y, T.sc[gg][1].z, T.sc[gg][1].w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const f32x4_t Sm = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, T.kr[gg][m]), qb[m],
                                                                f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // scale of token 4lq + i, block m: halfword 4i + m
        const uint32_t wv = sw[(4 * i + m) >> 1];
        const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)(((4 * i + m) & 1) ? (wv >> 16) : (wv & 0xFFFFu)));
        S[i] += d * Sm[i];
      }
    }
  }
  return S;
}

}  // namespace

template <int KV>
__global__ __launch_bounds__(256) void imp_stats_kernel(Params P, const uint16_t* __restrict__ q_obs, int n_obs,
                                                        const void* __restrict__ k_pool,
                                                        const int32_t* __restrict__ table, int max_blocks,
                                                        const int32_t* __restrict__ seq_lens,
                                                        float2* __restrict__ part) {
  __shared__ uint4 qs[kImpRows * 16];
  const int b = blockIdx.x, h = blockIdx.y, seq = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lq = lane >> 4, lc = lane & 15;
  const int L = seq_lens[seq], gsh = __builtin_ctz(P.g), n_rows = n_obs * P.g;
  const int n_sub = max_blocks * 4;  // partials per row: one per (block, wave)
  float2* out = part + ((size_t)seq * P.Hkv + h) * (size_t)n_rows * n_sub;
  const int v = b * kBlock < L ? table[(size_t)seq * max_blocks + b] : -1;
  if (v < 0) {  // a tile with no keys (past the sequence or unmapped)
    for (int x = tid; x < n_rows * 4; x += 256) out[(size_t)(x / 4) * n_sub + b * 4 + x % 4] = make_float2(-INFINITY, 0.f);
    return;
  }
  KTile<KV> kt;
  load_k_tile<KV>(k_pool, (size_t)v * P.Hkv + h, kt);
  const uint16_t* q_seq = q_obs + (size_t)seq * n_obs * P.Hq * kDim;
  for (int r0 = 0; r0 < n_rows; r0 += kImpRows) {
    if (r0 > 0) __syncthreads();  // every wave is done with the previous rows
    stage_q_rows(q_seq, h, gsh, P.Hq, n_rows, r0, qs);
    __syncthreads();
    const int n_rg = (min(kImpRows, n_rows - r0) + 15) / 16;
    for (int rg = 0; rg < n_rg; ++rg) {
      half8_t qb[4];
      q_rows_from_lds(qs, rg, qb);
      const int r = r0 + rg * 16 + lc;
      const int last = L - n_obs + (r < n_rows ? r >> gsh : 0);  // the row's own position: its last key
      // every key of the block precedes every observation query and all 16 rows exist: no masks
      const bool open = b * kBlock + kBlock - 1 <= L - n_obs && r0 + rg * 16 + 16 <= n_rows;
      float z[2][4], mx = -INFINITY;
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const f32x4_t S = imp_s<KV>(kt, qb, gg);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = b * kBlock + 32 * w + 16 * gg + 4 * lq + i;
          z[gg][i] = open || (r < n_rows && t <= last) ? S[i] * P.scale_log2 : -INFINITY;
          mx = fmaxf(mx, z[gg][i]);
        }
      }
      mx = fmaxf(mx, shfl_xor_f(mx, 16));
      mx = fmaxf(mx, shfl_xor_f(mx, 32));  // the wave's 32 tokens, row lc
      float sm = 0.f;
#pragma unroll
      for (int gg = 0; gg < 2; ++gg)
#pragma unroll
        for (int i = 0; i < 4; ++i) sm += exp2_diff(z[gg][i], mx);
      sm += shfl_xor_f(sm, 16);
      sm += shfl_xor_f(sm, 32);
      if (lq == 0 && r < n_rows) out[(size_t)r * n_sub + b * 4 + w] = make_float2(mx, sm);
    }
  }
}

// One workgroup per (sequence, KV head, row): M = max of the partial maxima, l = sum of
// exp2(m - M) * s, folded online -- (M, l) absorbs (m, s) as M' = max(M, m),
// l' = l exp2(M - M') + s exp2(m - M') -- with 8 loads in flight per lane, then across lanes and waves.
__device__ inline void ml_fold(float& M, float& l, float m, float s2) {
  const float Mn = fmaxf(M, m);
  l = l * exp2_diff(M, Mn) + s2 * exp2_diff(m, Mn);
  M = Mn;
}

__global__ __launch_bounds__(256) void imp_merge_kernel(const float2* __restrict__ part, int n_sub,
                                                        float2* __restrict__ stats) {
  __shared__ float2 red[4];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float2* p = part + (size_t)row * n_sub;
  float M = -INFINITY, l = 0.f;
  for (int x0 = tid; x0 < n_sub; x0 += 256 * 8) {
    float2 y[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) y[u] = p[min(x0 + 256 * u, n_sub - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (x0 + 256 * u < n_sub) ml_fold(M, l, y[u].x, y[u].y);
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) ml_fold(M, l, shfl_xor_f(M, m), shfl_xor_f(l, m));
  if (lane == 0) red[w] = make_float2(M, l);
  __syncthreads();
  if (tid == 0) {
    float Mt = red[0].x, lt = red[0].y;
    for (int k = 1; k < 4; ++k) ml_fold(Mt, lt, red[k].x, red[k].y);
    stats[row] = make_float2(Mt, lt);
  }
}

// dst: SEPARATE the importance itself [batch][Hkv][max_blocks * 128]; SHARED per-head rows of the
// same shape, summed by imp_sum_kernel.
template <int KV>
__global__ __launch_bounds__(256) void imp_accum_kernel(Params P, const uint16_t* __restrict__ q_obs, int n_obs,
                                                        const void* __restrict__ k_pool,
                                                        const int32_t* __restrict__ table, int max_blocks,
                                                        const int32_t* __restrict__ seq_lens,
                                                        const float2* __restrict__ stats,
                                                        float* __restrict__ dst) {
  __shared__ uint4 qs[kImpRows * 16];
  __shared__ float2 ls[kImpRows];
  const int b = blockIdx.x, h = blockIdx.y, seq = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lq = lane >> 4, lc = lane & 15;
  const int L = seq_lens[seq], gsh = __builtin_ctz(P.g), n_rows = n_obs * P.g;
  float* out = dst + ((size_t)seq * P.Hkv + h) * (size_t)max_blocks * kBlock + (size_t)b * kBlock;
  const int v = b * kBlock < L ? table[(size_t)seq * max_blocks + b] : -1;
  if (v < 0) {
    if (tid < kBlock) out[tid] = 0.f;
    return;
  }
  KTile<KV> kt;
  load_k_tile<KV>(k_pool, (size_t)v * P.Hkv + h, kt);
  const uint16_t* q_seq = q_obs + (size_t)seq * n_obs * P.Hq * kDim;
  const float2* st = stats + ((size_t)seq * P.Hkv + h) * n_rows;
  // lane (lc, lq) sums p over the rows lc + 16 * (row group) of token 4lq + i; the 16 lanes of a DPP
  // row are summed once, after every row group
  float acc[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  for (int r0 = 0; r0 < n_rows; r0 += kImpRows) {
    if (r0 > 0) __syncthreads();
    stage_q_rows(q_seq, h, gsh, P.Hq, n_rows, r0, qs);
    if (tid < kImpRows) ls[tid] = r0 + tid < n_rows ? st[r0 + tid] : make_float2(-INFINITY, 0.f);
    __syncthreads();
    const int n_rg = (min(kImpRows, n_rows - r0) + 15) / 16;
    for (int rg = 0; rg < n_rg; ++rg) {
      half8_t qb[4];
      q_rows_from_lds(qs, rg, qb);
      const int r = r0 + rg * 16 + lc;
      const float2 ml = ls[rg * 16 + lc];
      const float inv_l = ml.y > 0.f ? 1.0f / ml.y : 0.f;
      const int last = L - n_obs + (r < n_rows ? r >> gsh : 0);
      const bool open = b * kBlock + kBlock - 1 <= L - n_obs && r0 + rg * 16 + 16 <= n_rows;
      if (open) {  // no masks; the row's max is finite, so the logit is too
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          const f32x4_t S = imp_s<KV>(kt, qb, gg);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[gg][i] += fast_exp2(S[i] * P.scale_log2 - ml.x) * inv_l;
        }
      } else {
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          const f32x4_t S = imp_s<KV>(kt, qb, gg);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = b * kBlock + 32 * w + 16 * gg + 4 * lq + i;
            acc[gg][i] += r < n_rows && t <= last ? exp2_diff(S[i] * P.scale_log2, ml.x) * inv_l : 0.f;
          }
        }
      }
    }
  }
#pragma unroll
  for (int gg = 0; gg < 2; ++gg)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[gg][i] = row_sum16(acc[gg][i]);  // over the rows' lanes
  if (lc == 0) {
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
      for (int i = 0; i < 4; ++i) out[32 * w + 16 * gg + 4 * lq + i] = acc[gg][i];
  }
}

// SHARED: importance[seq][0][t] = sum over KV heads of the per-head rows.
__global__ __launch_bounds__(256) void imp_sum_kernel(const float* __restrict__ heads, int Hkv, size_t row_len,
                                                      float* __restrict__ imp) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int seq = blockIdx.y;
  if (t >= row_len) return;
  const float* src = heads + (size_t)seq * Hkv * row_len + t;
  float s = 0.f;
  for (int h = 0; h < Hkv; ++h) s += src[(size_t)h * row_len];
  imp[(size_t)seq * row_len + t] = s;
}

// One wave per (logical block, KV head, sequence): the rep_num best tokens of the block by score.
template <int KV>
__global__ __launch_bounds__(64) void dyn_reps_kernel(Params P, const void* __restrict__ k_pool,
                                                      const float* __restrict__ imp,
                                                      const int32_t* __restrict__ table, int max_blocks,
                                                      const int32_t* __restrict__ seq_lens,
                                                      uint16_t* __restrict__ rep_pool) {
  __shared__ float sc[kBlock];
  __shared__ int pick[kBlock];
  const int b = blockIdx.x, h = blockIdx.y, seq = blockIdx.z, lane = threadIdx.x;
  if ((b + 1) * kBlock > seq_lens[seq]) return;  // full blocks only
  const int v = table[(size_t)seq * max_blocks + b];
  if (v < 0) return;
  const float* row = imp + ((size_t)seq * P.G + (P.mode == kSeparate ? h : 0)) * (size_t)max_blocks * kBlock +
                     (size_t)b * kBlock;
  const float s0 = row[lane], s1 = row[lane + 64];
  sc[lane] = s0;
  sc[lane + 64] = s1;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int r0 = 0, r1 = 0;  // rank: how many tokens beat this one (higher score, or equal and lower)
  for (int t = 0; t < kBlock; ++t) {
    const float x = sc[t];
    r0 += x > s0 || (x == s0 && t < lane);
    r1 += x > s1 || (x == s1 && t < lane + 64);
  }
  const bool k0 = r0 < P.R, k1 = r1 < P.R;
  const unsigned long long m0 = __ballot(k0), m1 = __ballot(k1);
  const unsigned long long lt = (1ull << lane) - 1ull;
  if (k0) pick[__popcll(m0 & lt)] = lane;  // ascending token order
  if (k1) pick[__popcll(m0) + __popcll(m1 & lt)] = lane + 64;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint16_t* out = rep_pool + ((size_t)v * P.Hkv + h) * (size_t)P.R * kDim;
  const size_t tile = (size_t)v * P.Hkv + h;
  for (int i = lane >> 4; i < P.R; i += 4) {  // 16 lanes per row, 16 bytes each
    uint4 row8;
    if constexpr (KV == kKvFp16) {
      row8 = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(k_pool) + tile * kTile +
                                             (size_t)pick[i] * kDim + 8 * (lane & 15));
    } else {  // a quantized cache: the cached values, rounded to fp16 once
      constexpr int kRec = KV == kKvQ4 ? kQ4Record : KV == kKvI8 ? kI8Record : KV == kKvI4 ? kI4Record : kQ8Record;
      const unsigned char* rec = static_cast<const unsigned char*>(k_pool) + tile * (size_t)kRec;
      float f[8];
      if constexpr (KV == kKvQ4) q4_row8(rec, pick[i], lane & 15, f);
      else if constexpr (KV == kKvI8) i8_row8(rec, pick[i], lane & 15, f);
      else if constexpr (KV == kKvI4) i4_row8(rec, pick[i], lane & 15, f);
      else q8_row8(rec, pick[i], lane & 15, f);
      uint32_t wd[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) wd[e] = (uint32_t)f2h_bits(f[2 * e]) | ((uint32_t)f2h_bits(f[2 * e + 1]) << 16);
      row8 = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
    *reinterpret_cast<uint4*>(out + (size_t)i * kDim + 8 * (lane & 15)) = row8;
  }
}

hipError_t launch_token_importance(const Params& P, const void* q_obs, int n_obs, const void* k_pool,
                                   const int32_t* table, int max_blocks, const int32_t* seq_lens, int batch,
                                   float* imp, void* ws, hipStream_t s) {
  const size_t rows_all = (size_t)batch * P.Hkv * n_obs * P.g;
  const int n_sub = max_blocks * 4;
  float2* part = static_cast<float2*>(ws);
  float2* stats = part + rows_all * n_sub;
  float* heads = reinterpret_cast<float*>(stats + rows_all);  // SHARED only
  const uint16_t* q = static_cast<const uint16_t*>(q_obs);
  const dim3 tiles(max_blocks, P.Hkv, batch);
#define KVS_IMP_STATS(KV)                                                                                   \
  hipLaunchKernelGGL(imp_stats_kernel<KV>, tiles, dim3(256), 0, s, P, q, n_obs, k_pool, table, max_blocks, \
                     seq_lens, part)
  switch (P.kv) {
    case kKvQ8: KVS_IMP_STATS(kKvQ8); break;
    case kKvQ4: KVS_IMP_STATS(kKvQ4); break;
    case kKvI8: KVS_IMP_STATS(kKvI8); break;
    case kKvI4: KVS_IMP_STATS(kKvI4); break;
    default: KVS_IMP_STATS(kKvFp16); break;
  }
#undef KVS_IMP_STATS
  hipLaunchKernelGGL(imp_merge_kernel, dim3((unsigned)rows_all), dim3(256), 0, s, part, n_sub, stats);
  const bool shared = P.mode == kShared;
  float* dst = shared ? heads : imp;
#define KVS_IMP_ACCUM(KV)                                                                                   \
  hipLaunchKernelGGL(imp_accum_kernel<KV>, tiles, dim3(256), 0, s, P, q, n_obs, k_pool, table, max_blocks, \
                     seq_lens, stats, dst)
  switch (P.kv) {
    case kKvQ8: KVS_IMP_ACCUM(kKvQ8); break;
    case kKvQ4: KVS_IMP_ACCUM(kKvQ4); break;
    case kKvI8: KVS_IMP_ACCUM(kKvI8); break;
    case kKvI4: KVS_IMP_ACCUM(kKvI4); break;
    default: KVS_IMP_ACCUM(kKvFp16); break;
  }
#undef KVS_IMP_ACCUM
  if (shared) {
    const size_t row_len = (size_t)max_blocks * kBlock;
    hipLaunchKernelGGL(imp_sum_kernel, dim3((unsigned)((row_len + 255) / 256), batch), dim3(256), 0, s, heads,
                       P.Hkv, row_len, imp);
  }
  return hipGetLastError();
}

size_t token_importance_ws_bytes(const Params& P, int batch, int max_blocks, int n_obs) {
  const size_t rows = (size_t)batch * P.Hkv * n_obs * P.g;
  return rows * max_blocks * 4 * sizeof(float2) + rows * sizeof(float2) +
         (size_t)batch * P.Hkv * max_blocks * kBlock * sizeof(float);
}

hipError_t launch_dynamic_reps(const Params& P, const void* k_pool, const float* imp, const int32_t* table,
                               int max_blocks, const int32_t* seq_lens, int batch, void* rep_pool,
                               hipStream_t s) {
  const dim3 grid(max_blocks, P.Hkv, batch);
  uint16_t* rp = static_cast<uint16_t*>(rep_pool);
  switch (P.kv) {
    case kKvQ8: hipLaunchKernelGGL(dyn_reps_kernel<kKvQ8>, grid, dim3(64), 0, s, P, k_pool, imp, table, max_blocks, seq_lens, rp); break;
    case kKvQ4: hipLaunchKernelGGL(dyn_reps_kernel<kKvQ4>, grid, dim3(64), 0, s, P, k_pool, imp, table, max_blocks, seq_lens, rp); break;
    case kKvI8: hipLaunchKernelGGL(dyn_reps_kernel<kKvI8>, grid, dim3(64), 0, s, P, k_pool, imp, table, max_blocks, seq_lens, rp); break;
    case kKvI4: hipLaunchKernelGGL(dyn_reps_kernel<kKvI4>, grid, dim3(64), 0, s, P, k_pool, imp, table, max_blocks, seq_lens, rp); break;
    default: hipLaunchKernelGGL(dyn_reps_kernel<kKvFp16>, grid, dim3(64), 0, s, P, k_pool, imp, table, max_blocks, seq_lens, rp); break;
  }
  return hipGetLastError();
}

}  // namespace kvs
