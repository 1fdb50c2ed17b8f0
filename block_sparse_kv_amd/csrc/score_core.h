// Block scoring for one workgroup of 256 lanes (used by kvs_score_blocks and kvs_decode_step).
// KTransformers long-context sparse attention (lmnt.cn): §3.1 Quest upper bound
// sum_c max(q_c*kmax_c, q_c*kmin_c); §4.3 similarity of the query with the reps; §4.5 SEPARATE /
// SHARED head selection.
//
// Lane layout: 16 lanes (one DPP row) per (logical block, KV head); lane c owns channels 8c..8c+7 and
// keeps the matching slice of the g query heads of its KV head in registers.  256 lanes cover
// 16/Hkv blocks x Hkv heads per pass (or, PER_HEAD, 16 blocks of one KV head); 4 passes are issued
// together (table entries first, then all rep loads) so one workgroup pays the memory latency about
// twice, not once per pass.  Reps are read
// with 128-bit loads (a 16-lane row reads one 256 B fp16 rep row).  For the linear reps (Max, Mean,
// Fix) the g query heads are summed first, since sum_j q_j.rep = (sum_j q_j).rep; Quest is per head
// (the max is not linear).  Quest's max(q_c*kmax_c, q_c*kmin_c) is q_c*kmax_c where q_c >= 0 and
// q_c*kmin_c where q_c < 0 (kmin_c <= kmax_c), so each lane splits its fp16 query pairs once by sign
// (the other half zeroed) and a block costs two 2-wide fp16 dot products with fp32 accumulation
// (v_dot2_f32_f16) per channel pair and head: the fp16 products are exact in fp32, and each pair of
// them is added to the sum with one rounding.
#pragma once

#include "kvs_device.h"

namespace kvs {

constexpr int kScorePasses = 4;  // passes whose loads are in flight together

// Blocks one scoring workgroup covers: kScorePasses passes of 16/Hkv blocks (all KV heads), or of 16
// blocks (one KV head).
__host__ __device__ inline int score_blocks_per_wg(const Params& P) { return (16 / P.Hkv) * kScorePasses; }
constexpr int kScoreBlocksPerHeadWg = 16 * kScorePasses;

// Scores of logical blocks [b0, b0 + nb) of one sequence (cache length L): of every KV head, or with
// PER_HEAD (SEPARATE only) of KV head h_one.  Non-candidates get -INFINITY.  scores_row: SEPARATE ->
// [Hkv][max_blocks] rows of this sequence, SHARED -> [max_blocks].  COH: the scores are stored for a
// workgroup of the same kernel (st_coh).
// lds_chunk (PER_HEAD, nullable): also receives every block's score (-inf for non-candidates and past
// the row) at [block - b0] and its physical id (0 for non-candidates) as an int at [64 + block - b0],
// for the workgroup's own use after a barrier (nb <= 64).
// LIST: [b0, b0 + nb) are positions in the list ids[0..n_list) of logical block ids (-1 or any id
// outside the candidates: not a candidate); the scores go to position-indexed rows of n_list entries
// (scores_row[(PER_HEAD ? h : 0) * n_list + position]), and each candidate's physical id, coherently,
// to phys_row at the same index.
template <int G, int METHOD, int MODE, bool PER_HEAD = false, bool COH = false, bool LIST = false>
__device__ __forceinline__ void score_blocks_range(const Params& P, const uint16_t* __restrict__ q_seq,
                                          const void* __restrict__ rep_pool,
                                          const int32_t* __restrict__ trow, int max_blocks, int L,
                                          int b0, int nb, float* __restrict__ scores_row,
                                          float* lds_part /* >= 16 * kScorePasses floats */,
                                          int h_one = 0, float* lds_chunk = nullptr,
                                          const int32_t* __restrict__ ids = nullptr, int n_list = 0,
                                          int32_t* __restrict__ phys_row = nullptr) {
  static_assert(!(PER_HEAD && MODE == kShared), "a SHARED score sums over every KV head");
  static_assert(!(LIST && !COH), "list scores are handed to the selecting workgroup");
  const int n_row = LIST ? n_list : max_blocks;  // entries of a score row
  const int Hkv = P.Hkv;
  const int t = threadIdx.x, c = t & 15;
  const int h = PER_HEAD ? h_one : (t >> 4) % Hkv;
  const int bpp = PER_HEAD ? 16 : 16 / Hkv;  // blocks per pass
  const int slot = PER_HEAD ? t >> 4 : (t >> 4) / Hkv;
  const Regions rg = regions_of(L, P.initial_len, P.local_len);
  constexpr int RMAX = METHOD == kQuest ? 2 : (METHOD == kMean ? 2 : 1);  // 16-byte loads per pass

  typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
  const uint16_t* qh = q_seq + (size_t)h * G * kDim + c * 8;
  uint32_t qpos[G][4], qneg[G][4];  // Quest: the g query heads' fp16 pairs split by sign
  float qs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // linear reps: the g query heads summed
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const uint4 w = *reinterpret_cast<const uint4*>(qh + j * kDim);
    if constexpr (METHOD == kQuest) {
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t m = ((ws[i] >> 15) & 0x00010001u) * 0xFFFFu;  // the negative halves
        qneg[j][i] = ws[i] & m;
        qpos[j][i] = ws[i] & ~m;
      }
    } else {
      float qf[8];
      unpack8(w, qf);
#pragma unroll
      for (int e = 0; e < 8; ++e) qs[e] += qf[e];
    }
  }

  // Loads that must be in flight together are issued without branches: indices are clamped to valid
  // ones (a non-candidate reads physical block 0) and the results are masked afterwards, so the
  // compiler places no wait between them.
  for (int base = b0; base < b0 + nb; base += bpp * kScorePasses) {
    int blk[kScorePasses];  // row position: the logical block, or with LIST the list position
    int lb[kScorePasses];   // logical block
    bool inr[kScorePasses], cand[kScorePasses];
    size_t phys[kScorePasses];
#pragma unroll
    for (int p = 0; p < kScorePasses; ++p) {
      blk[p] = base + p * bpp + slot;
      inr[p] = blk[p] < b0 + nb && blk[p] < n_row;
    }
    if constexpr (LIST) {
#pragma unroll
      for (int p = 0; p < kScorePasses; ++p) lb[p] = ids[min(blk[p], n_row - 1)];
    } else {
#pragma unroll
      for (int p = 0; p < kScorePasses; ++p) lb[p] = blk[p];
    }
#pragma unroll
    for (int p = 0; p < kScorePasses; ++p) {
      cand[p] = inr[p] && lb[p] >= rg.cand_lo && lb[p] < rg.cand_hi && lb[p] < max_blocks;
      const int t = trow[min(max(lb[p], 0), max_blocks - 1)];
      phys[p] = cand[p] ? (size_t)t : 0;
    }
    uint4 raw[kScorePasses][RMAX];
#pragma unroll
    for (int p = 0; p < kScorePasses; ++p) {
      if constexpr (METHOD == kQuest) {
        const uint16_t* rp = static_cast<const uint16_t*>(rep_pool) + (phys[p] * Hkv + h) * 2 * kDim + c * 8;
        raw[p][0] = ld_stream16(rp);
        raw[p][1] = ld_stream16(rp + kDim);
      } else if constexpr (METHOD == kMean) {
        const float* rp = static_cast<const float*>(rep_pool) + (phys[p] * Hkv + h) * kDim + c * 8;
        raw[p][0] = ld_stream16(rp);
        raw[p][RMAX - 1] = ld_stream16(rp + 4);
      } else {
        const uint16_t* rp = static_cast<const uint16_t*>(rep_pool) + (phys[p] * Hkv + h) * (size_t)P.R * kDim + c * 8;
        raw[p][0] = ld_stream16(rp);
      }
    }
    float acc[kScorePasses];
#pragma unroll
    for (int p = 0; p < kScorePasses; ++p) {
      acc[p] = 0.f;
      if constexpr (METHOD == kQuest) {
        const uint32_t kmin[4] = {raw[p][0].x, raw[p][0].y, raw[p][0].z, raw[p][0].w};
        const uint32_t kmax[4] = {raw[p][1].x, raw[p][1].y, raw[p][1].z, raw[p][1].w};
#pragma unroll
        for (int j = 0; j < G; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[p] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, qpos[j][i]),
                                            __builtin_bit_cast(h2_t, kmax[i]), acc[p], false);
            acc[p] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, qneg[j][i]),
                                            __builtin_bit_cast(h2_t, kmin[i]), acc[p], false);
          }
      } else {
        float rs[8];
        if constexpr (METHOD == kMean) {
          const uint4 x0 = raw[p][0], x1 = raw[p][RMAX - 1];
          rs[0] = __uint_as_float(x0.x); rs[1] = __uint_as_float(x0.y);
          rs[2] = __uint_as_float(x0.z); rs[3] = __uint_as_float(x0.w);
          rs[4] = __uint_as_float(x1.x); rs[5] = __uint_as_float(x1.y);
          rs[6] = __uint_as_float(x1.z); rs[7] = __uint_as_float(x1.w);
        } else {
          unpack8(raw[p][0], rs);
          const uint16_t* rp = static_cast<const uint16_t*>(rep_pool) + (phys[p] * Hkv + h) * (size_t)P.R * kDim + c * 8;
          for (int r0 = 1; r0 < P.R; r0 += 8) {  // Fix: sum of the rep rows (8 loads in flight), then one dot
            uint4 x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) x[u] = ld_stream16(rp + (size_t)(r0 + u < P.R ? r0 + u : 0) * kDim);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              float f[8];
              unpack8(x[u], f);
              const bool ok = r0 + u < P.R;
#pragma unroll
              for (int e = 0; e < 8; ++e) rs[e] += ok ? f[e] : 0.f;
            }
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[p] += qs[e] * rs[e];
      }
    }
#pragma unroll
    for (int p = 0; p < kScorePasses; ++p) acc[p] = row_sum16(acc[p]);

    if constexpr (MODE == kSeparate) {
      if (c == 0) {
#pragma unroll
        for (int p = 0; p < kScorePasses; ++p) {
          if (PER_HEAD && lds_chunk) {
            lds_chunk[blk[p] - b0] = cand[p] ? acc[p] : -INFINITY;
            reinterpret_cast<int*>(lds_chunk)[64 + blk[p] - b0] = (int)phys[p];
          }
          if (!inr[p]) continue;
          float* dst = scores_row + (size_t)h * n_row + blk[p];
          const float v = cand[p] ? acc[p] : -INFINITY;
          if constexpr (COH) st_coh(dst, v); else *dst = v;
          if constexpr (LIST) st_coh(phys_row + (size_t)h * n_row + blk[p], (int32_t)phys[p]);
        }
      }
    } else {
      if (c == 0) {
#pragma unroll
        for (int p = 0; p < kScorePasses; ++p) lds_part[p * 16 + slot * Hkv + h] = acc[p];
      }
      __syncthreads();
      if (c == 0 && h == 0) {
#pragma unroll
        for (int p = 0; p < kScorePasses; ++p) {
          if (!inr[p]) continue;
          float s = 0.f;
          for (int hh = 0; hh < Hkv; ++hh) s += lds_part[p * 16 + slot * Hkv + hh];
          const float v = cand[p] ? s : -INFINITY;
          if constexpr (COH) st_coh(scores_row + blk[p], v); else scores_row[blk[p]] = v;
          if constexpr (LIST) st_coh(phys_row + blk[p], (int32_t)phys[p]);
        }
      }
      __syncthreads();
    }
  }
}

}  // namespace kvs
