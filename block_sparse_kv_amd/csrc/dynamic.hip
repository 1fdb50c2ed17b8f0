// Dynamic reps: every cached token's cumulative attention score, and each block's top tokens as its
// reps.  The KTransformers long-context article (§4.3, rep table) names the method -- each token's
// accumulated attention score, the highest-scoring tokens of a block become its reps -- and leaves
// the scoring method open.  Here a token's score is the attention it receives from the n_obs
// observation queries (the last n_obs tokens of the cache, each attending causally, scale
// 1/sqrt(d)), summed over those queries and the query heads of the selection group.
//
// The probabilities need each query row's softmax normaliser over all of its keys, so three passes:
//  1. imp_stats_kernel, one workgroup per (block, KV head, sequence): S = K Q^T on the matrix cores
//     for every row (observation query, query head of the KV head), 16 rows at a time, K in the
//     A-operand layout straight from HBM (loaded once per tile); per row the tile's max and sum of
//     exp2 in the exp2 domain -> partials [seq][h][row][block].
//  2. imp_merge_kernel, one wave per (sequence, KV head, row): log-sum-exp of the row's partials.
//  3. imp_accum_kernel, one workgroup per (block, sequence): for every KV head the same products
//     again, p = exp2(z - M) / l summed over the rows of a DPP row of 16 lanes, then over row groups
//     and (SHARED) KV heads in registers, and each token's total stored once.
// dyn_reps_kernel: one wave per (block, KV head, sequence) ranks the block's 128 scores by counting
// (higher score, or equal and lower token, beats) and copies the K rows of the rep_num best, in
// ascending token order, into the rep pool; a Dynamic block is then scored like Fix.
#include "attn_core.h"
#include "kvs_launch.h"

namespace kvs {

namespace {

// K tile of (phys, h) in the A-operand layout of attn_tile: lane (lc, lq) of wave w, token group g
// (16 tokens), MFMA m: token 32w + 16g + lc, channels 32m + 8lq .. +8.
__device__ inline void load_k_tile(const uint16_t* __restrict__ k_pool, size_t tile, uint4 (&kr)[2][4]) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lq = lane >> 4, lc = lane & 15;
  const uint16_t* Kt = k_pool + tile * kTile;
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int m = 0; m < 4; ++m) kr[g][m] = ld_stream16(Kt + (32 * w + 16 * g + lc) * kDim + 32 * m + 8 * lq);
}

// Q^T B operand of rows rg*16 .. +16 of KV head h: row r = observation i * g + head j of the group;
// lane (lc, lq) holds row lc, channels 32m + 8lq .. +8.  Rows past n_rows are zero.
__device__ inline void load_q_rows(const uint16_t* __restrict__ q_seq, int h, int g, int Hq, int n_rows,
                                   int rg, half8_t (&qb)[4]) {
  const int lane = threadIdx.x & 63, lq = lane >> 4, lc = lane & 15;
  const int r = rg * 16 + lc;
  const bool ok = r < n_rows;
  const int rr = ok ? r : 0;
  const uint16_t* qr = q_seq + ((size_t)(rr / g) * Hq + h * g + rr % g) * kDim;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint4 v = *reinterpret_cast<const uint4*>(qr + 32 * m + 8 * lq);
    qb[m] = __builtin_bit_cast(half8_t, ok ? v : make_uint4(0, 0, 0, 0));
  }
}

}  // namespace

__global__ __launch_bounds__(256) void imp_stats_kernel(Params P, const uint16_t* __restrict__ q_obs, int n_obs,
                                                        const uint16_t* __restrict__ k_pool,
                                                        const int32_t* __restrict__ table, int max_blocks,
                                                        const int32_t* __restrict__ seq_lens,
                                                        float2* __restrict__ part) {
  __shared__ float red[4][16];
  const int b = blockIdx.x, h = blockIdx.y, seq = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lq = lane >> 4, lc = lane & 15;
  const int L = seq_lens[seq], g = P.g, n_rows = n_obs * g, n_rg = (n_rows + 15) / 16;
  float2* out = part + ((size_t)seq * P.Hkv + h) * (size_t)n_rows * max_blocks;
  const int v = b * kBlock < L ? table[(size_t)seq * max_blocks + b] : -1;
  if (v < 0) {  // a tile with no keys (past the sequence or unmapped)
    for (int r = tid; r < n_rows; r += 256) out[(size_t)r * max_blocks + b] = make_float2(-INFINITY, 0.f);
    return;
  }
  uint4 kr[2][4];
  load_k_tile(k_pool, (size_t)v * P.Hkv + h, kr);
  const uint16_t* q_seq = q_obs + (size_t)seq * n_obs * P.Hq * kDim;
  for (int rg = 0; rg < n_rg; ++rg) {
    half8_t qb[4];
    load_q_rows(q_seq, h, g, P.Hq, n_rows, rg, qb);
    const int r = rg * 16 + lc;
    const int last = L - n_obs + (r < n_rows ? r / g : 0);  // the row's own position: its last key
    float z[2][4], mx = -INFINITY;
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      f32x4_t S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 4; ++m)
        S = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, kr[gg][m]), qb[m], S, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = b * kBlock + 32 * w + 16 * gg + 4 * lq + i;
        z[gg][i] = r < n_rows && t <= last ? S[i] * P.scale_log2 : -INFINITY;
        mx = fmaxf(mx, z[gg][i]);
      }
    }
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    if (lq == 0) red[w][lc] = mx;
    __syncthreads();
    const float tm = fmaxf(fmaxf(red[0][lc], red[1][lc]), fmaxf(red[2][lc], red[3][lc]));
    __syncthreads();
    float sm = 0.f;
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm += exp2_diff(z[gg][i], tm);
    sm += shfl_xor_f(sm, 16);
    sm += shfl_xor_f(sm, 32);
    if (lq == 0) red[w][lc] = sm;
    __syncthreads();
    if (tid < 16 && rg * 16 + tid < n_rows)
      out[(size_t)(rg * 16 + tid) * max_blocks + b] =
          make_float2(tm, (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]));
    __syncthreads();
  }
}

// One wave per (sequence, KV head, row): M = max of the partial maxima, l = sum of exp2(m - M) * s.
__global__ __launch_bounds__(256) void imp_merge_kernel(const float2* __restrict__ part, int n_rows_all,
                                                        int max_blocks, float2* __restrict__ stats) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= n_rows_all) return;
  const float2* p = part + (size_t)row * max_blocks;
  float M = -INFINITY;
  for (int b = lane; b < max_blocks; b += 64) M = fmaxf(M, p[b].x);
  M = wave_max_f32(M);
  float l = 0.f;
  for (int b = lane; b < max_blocks; b += 64) {
    const float2 x = p[b];
    l += x.y * exp2_diff(x.x, M);
  }
  l = wave_sum_f32(l);
  if (lane == 0) stats[row] = make_float2(M, l);
}

__global__ __launch_bounds__(256) void imp_accum_kernel(Params P, const uint16_t* __restrict__ q_obs, int n_obs,
                                                        const uint16_t* __restrict__ k_pool,
                                                        const int32_t* __restrict__ table, int max_blocks,
                                                        const int32_t* __restrict__ seq_lens,
                                                        const float2* __restrict__ stats,
                                                        float* __restrict__ imp) {
  const int b = blockIdx.x, seq = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lq = lane >> 4, lc = lane & 15;
  const int L = seq_lens[seq], g = P.g, n_rows = n_obs * g, n_rg = (n_rows + 15) / 16;
  const size_t row_len = (size_t)max_blocks * kBlock;
  const int v = b * kBlock < L ? table[(size_t)seq * max_blocks + b] : -1;
  const uint16_t* q_seq = q_obs + (size_t)seq * n_obs * P.Hq * kDim;
  float acc[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  for (int h = 0; h < P.Hkv; ++h) {
    if (v >= 0) {
      uint4 kr[2][4];
      load_k_tile(k_pool, (size_t)v * P.Hkv + h, kr);
      const float2* st = stats + ((size_t)seq * P.Hkv + h) * n_rows;
      for (int rg = 0; rg < n_rg; ++rg) {
        half8_t qb[4];
        load_q_rows(q_seq, h, g, P.Hq, n_rows, rg, qb);
        const int r = rg * 16 + lc;
        const float2 ml = st[r < n_rows ? r : 0];
        const float inv_l = ml.y > 0.f ? 1.0f / ml.y : 0.f;
        const int last = L - n_obs + (r < n_rows ? r / g : 0);
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          f32x4_t S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int m = 0; m < 4; ++m)
            S = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, kr[gg][m]), qb[m], S, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = b * kBlock + 32 * w + 16 * gg + 4 * lq + i;
            const float p = r < n_rows && t <= last ? exp2_diff(S[i] * P.scale_log2, ml.x) * inv_l : 0.f;
            acc[gg][i] += row_sum16(p);  // the 16 rows of this group (one DPP row = one token)
          }
        }
      }
    }
    if (P.mode == kSeparate || h == P.Hkv - 1) {  // one score row per KV head, or one for all
      if (lc == 0) {
        float* dst = imp + ((size_t)seq * P.G + (P.mode == kSeparate ? h : 0)) * row_len + (size_t)b * kBlock;
#pragma unroll
        for (int gg = 0; gg < 2; ++gg)
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[32 * w + 16 * gg + 4 * lq + i] = acc[gg][i];
      }
#pragma unroll
      for (int gg = 0; gg < 2; ++gg)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[gg][i] = 0.f;
    }
  }
}

// One wave per (logical block, KV head, sequence): the rep_num best tokens of the block by score.
__global__ __launch_bounds__(64) void dyn_reps_kernel(Params P, const uint16_t* __restrict__ k_pool,
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
  const uint16_t* Kt = k_pool + ((size_t)v * P.Hkv + h) * kTile;
  uint16_t* out = rep_pool + ((size_t)v * P.Hkv + h) * (size_t)P.R * kDim;
  for (int i = lane >> 4; i < P.R; i += 4)  // 16 lanes per row, 16 bytes each
    *reinterpret_cast<uint4*>(out + (size_t)i * kDim + 8 * (lane & 15)) =
        *reinterpret_cast<const uint4*>(Kt + (size_t)pick[i] * kDim + 8 * (lane & 15));
}

hipError_t launch_token_importance(const Params& P, const void* q_obs, int n_obs, const void* k_pool,
                                   const int32_t* table, int max_blocks, const int32_t* seq_lens, int batch,
                                   float* imp, void* ws, hipStream_t s) {
  const int n_rows = n_obs * P.g;
  float2* part = static_cast<float2*>(ws);
  float2* stats = part + (size_t)batch * P.Hkv * n_rows * max_blocks;
  const uint16_t* q = static_cast<const uint16_t*>(q_obs);
  const uint16_t* kp = static_cast<const uint16_t*>(k_pool);
  hipLaunchKernelGGL(imp_stats_kernel, dim3(max_blocks, P.Hkv, batch), dim3(256), 0, s, P, q, n_obs, kp, table,
                     max_blocks, seq_lens, part);
  const int rows_all = batch * P.Hkv * n_rows;
  hipLaunchKernelGGL(imp_merge_kernel, dim3((rows_all + 3) / 4), dim3(256), 0, s, part, rows_all, max_blocks, stats);
  hipLaunchKernelGGL(imp_accum_kernel, dim3(max_blocks, batch), dim3(256), 0, s, P, q, n_obs, kp, table,
                     max_blocks, seq_lens, stats, imp);
  return hipGetLastError();
}

size_t token_importance_ws_bytes(const Params& P, int batch, int max_blocks, int n_obs) {
  const size_t rows = (size_t)batch * P.Hkv * n_obs * P.g;
  return rows * max_blocks * sizeof(float2) + rows * sizeof(float2);
}

hipError_t launch_dynamic_reps(const Params& P, const void* k_pool, const float* imp, const int32_t* table,
                               int max_blocks, const int32_t* seq_lens, int batch, void* rep_pool,
                               hipStream_t s) {
  hipLaunchKernelGGL(dyn_reps_kernel, dim3(max_blocks, P.Hkv, batch), dim3(64), 0, s, P,
                     static_cast<const uint16_t*>(k_pool), imp, table, max_blocks, seq_lens,
                     static_cast<uint16_t*>(rep_pool));
  return hipGetLastError();
}

}  // namespace kvs
