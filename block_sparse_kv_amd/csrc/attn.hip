// kvs_sparse_decode_attn kernels: exact softmax attention over the retrieved cache
// (KTransformers long-context sparse attention, lmnt.cn: §4.2 Initial and Local always attended,
// selected Context blocks in between; §4.6 attn(query, kvcache_after_retrieval), logits scaled by
// 1/sqrt(head_dim)).
//
// Split flash-decoding.  The attended tiles of one (sequence, KV head) -- Initial tiles, the selected
// tiles, the Local tiles -- form one list; workgroup (split, h, seq) takes `tps` consecutive tiles of
// it and all g query heads that read KV head h.  Each of its 4 waves owns 32 token rows of every tile:
// lane (r = lane/16, c = lane%16) loads channels 8c..8c+7 of tokens 32w + 4i + r, i = 0..7, so each
// wave-wide 128-bit load is 4 whole token rows (1 KiB contiguous).  q.k is a packed fp16 dot product
// accumulated in fp32 and summed across the 16-lane DPP row; softmax runs online in the exp2 domain per
// (wave, row) stream; P.V accumulates in fp32.  Streams are folded across rows (lane shuffles) and
// waves (LDS) and the split's (max, sum, unnormalised output) goes to the workspace; the merge kernel
// combines splits by log-sum-exp.
#include "kvs_device.h"
#include "kvs_launch.h"

namespace kvs {

template <int G>
__global__ __launch_bounds__(256) void attn_split_kernel(
    Params P, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, const int32_t* __restrict__ table, int max_blocks,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ sel_count, int tps, int n_splits, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  const int split = blockIdx.x, h = blockIdx.y, seq = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r = lane >> 4, c = lane & 15;
  const int L = seq_lens[seq];
  const int grp = P.mode == kSeparate ? h : 0;
  const size_t grow = (size_t)seq * P.G + grp;
  const Regions rg = regions_of(L, P.initial_len, P.local_len);
  const int k_sel = L > rg.init_end ? sel_count[grow] : 0;
  const TileList tl = tiles_of(L, P, k_sel);
  const int nT = tl.count();
  const int t0 = split * tps;
  if (t0 >= nT) return;
  const int t1 = min(nT, t0 + tps);
  const int32_t* trow = table + (size_t)seq * max_blocks;
  const int32_t* srow = sel + grow * P.topk;

  half2_t q2[G][4];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const uint4 v = *reinterpret_cast<const uint4*>(q + ((size_t)seq * P.Hq + (size_t)h * G + j) * kDim + c * 8);
    q2[j][0] = __builtin_bit_cast(half2_t, v.x);
    q2[j][1] = __builtin_bit_cast(half2_t, v.y);
    q2[j][2] = __builtin_bit_cast(half2_t, v.z);
    q2[j][3] = __builtin_bit_cast(half2_t, v.w);
  }
  float m[G], l[G], o[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY; l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[j][e] = 0.f;
  }

  for (int ti = t0; ti < t1; ++ti) {
    int lb, ntok;
    if (ti < tl.nI) { lb = ti; ntok = min(kBlock, L - lb * kBlock); }
    else if (ti < tl.nI + tl.k) { lb = srow[ti - tl.nI]; ntok = kBlock; }
    else { lb = tl.loc_b0 + (ti - tl.nI - tl.k); ntok = min(kBlock, L - lb * kBlock); }
    const size_t off = ((size_t)trow[lb] * P.Hkv + h) * kTile + (size_t)c * 8;
    const uint16_t* Kt = k_pool + off;
    const uint16_t* Vt = v_pool + off;
    uint4 kr[8], vr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tok = 32 * w + 4 * i + r;
      if (tok < ntok) {
        kr[i] = ld_stream16(Kt + tok * kDim);
        vr[i] = ld_stream16(Vt + tok * kDim);
      } else {
        kr[i] = make_uint4(0, 0, 0, 0);
        vr[i] = make_uint4(0, 0, 0, 0);
      }
    }
    float vf[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) unpack8(vr[i], vf[i]);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float s[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float a = __builtin_amdgcn_fdot2(q2[j][0], __builtin_bit_cast(half2_t, kr[i].x), 0.f, false);
        a = __builtin_amdgcn_fdot2(q2[j][1], __builtin_bit_cast(half2_t, kr[i].y), a, false);
        a = __builtin_amdgcn_fdot2(q2[j][2], __builtin_bit_cast(half2_t, kr[i].z), a, false);
        a = __builtin_amdgcn_fdot2(q2[j][3], __builtin_bit_cast(half2_t, kr[i].w), a, false);
        s[i] = row_sum16(a);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int tok = 32 * w + 4 * i + r;
        s[i] = tok < ntok ? s[i] * P.scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[i]);
      }
      const float mn = fmaxf(m[j], mx);
      if (mn == -INFINITY) continue;  // this row holds no token of the tile
      const float alpha = exp2_diff(m[j], mn);
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[j][e] *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = fast_exp2(s[i] - mn);
        ps += p;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[j][e] += p * vf[i][e];
      }
      l[j] = l[j] * alpha + ps;
      m[j] = mn;
    }
  }

  // fold the 4 row streams of this wave
#pragma unroll
  for (int msk = 16; msk <= 32; msk <<= 1) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float mo = shfl_xor_f(m[j], msk), lo = shfl_xor_f(l[j], msk);
      const float mn = fmaxf(m[j], mo);
      const float a = exp2_diff(m[j], mn), b = exp2_diff(mo, mn);
      l[j] = l[j] * a + lo * b;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[j][e] = o[j][e] * a + shfl_xor_f(o[j][e], msk) * b;
      m[j] = mn;
    }
  }
  // fold the 4 waves through LDS and write this split's partial
  __shared__ float sm[4][G], sl[4][G], so[4][G][kDim];
  if (r == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
      for (int e = 0; e < 8; ++e) so[w][j][c * 8 + e] = o[j][e];
      if (c == 0) { sm[w][j] = m[j]; sl[w][j] = l[j]; }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * kDim; idx += 256) {
    const int j = idx / kDim, ch = idx % kDim;
    const float M = fmaxf(fmaxf(sm[0][j], sm[1][j]), fmaxf(sm[2][j], sm[3][j]));
    float lsum = 0.f, acc = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float f = exp2_diff(sm[ww][j], M);
      lsum += sl[ww][j] * f;
      acc += so[ww][j][ch] * f;
    }
    const size_t pr = ((size_t)seq * P.Hq + (size_t)h * G + j) * n_splits + split;
    part_o[pr * kDim + ch] = acc;
    if (ch == 0) { part_ml[pr * 2] = M; part_ml[pr * 2 + 1] = lsum; }
  }
}

// One workgroup of 128 lanes (one per channel) per (query head, sequence).
__global__ __launch_bounds__(128) void attn_merge_kernel(Params P, const int32_t* __restrict__ seq_lens,
                                                         const int32_t* __restrict__ sel_count,
                                                         int tps, int n_splits,
                                                         const float* __restrict__ part_o,
                                                         const float* __restrict__ part_ml,
                                                         float* __restrict__ out) {
  const int j = blockIdx.x, seq = blockIdx.y, ch = threadIdx.x;
  const int h = j / P.g;
  const int grp = P.mode == kSeparate ? h : 0;
  const int L = seq_lens[seq];
  const Regions rg = regions_of(L, P.initial_len, P.local_len);
  const int k_sel = L > rg.init_end ? sel_count[(size_t)seq * P.G + grp] : 0;
  const int nT = tiles_of(L, P, k_sel).count();
  const int ns = (nT + tps - 1) / tps;
  const size_t pr0 = ((size_t)seq * P.Hq + j) * n_splits;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, part_ml[(pr0 + s) * 2]);
  float lsum = 0.f, acc = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float f = exp2_diff(part_ml[(pr0 + s) * 2], M);
    lsum += part_ml[(pr0 + s) * 2 + 1] * f;
    acc += part_o[(pr0 + s) * kDim + ch] * f;
  }
  out[((size_t)seq * P.Hq + j) * kDim + ch] = lsum > 0.f ? acc / lsum : 0.f;
}

AttnPlan attn_plan(const Params& P, int batch, int max_blocks) {
  const int nI = (P.initial_len + kBlock - 1) / kBlock;
  const int nLoc = (P.local_len + 2 * kBlock - 2) / kBlock;
  long maxT = (long)nI + P.topk + nLoc;
  if (maxT > max_blocks) maxT = max_blocks;
  if (maxT < 1) maxT = 1;
  const long total = (long)batch * P.Hkv * maxT;
  long tps = total / 1536;
  if (tps < 1) tps = 1;
  if (tps > 32) tps = 32;
  AttnPlan a;
  a.tps = (int)tps;
  a.n_splits = (int)((maxT + tps - 1) / tps);
  a.part_o_bytes = (size_t)batch * P.Hq * a.n_splits * kDim * sizeof(float);
  a.part_ml_bytes = (size_t)batch * P.Hq * a.n_splits * 2 * sizeof(float);
  return a;
}

hipError_t launch_attn(const Params& P, const AttnPlan& A, const void* q, const void* k_pool,
                       const void* v_pool, const int32_t* table, int max_blocks,
                       const int32_t* seq_lens, int batch, const int32_t* sel,
                       const int32_t* sel_count, float* out, float* part_o, float* part_ml,
                       hipStream_t s) {
  const dim3 grid(A.n_splits, P.Hkv, batch), block(256);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kp = static_cast<const uint16_t*>(k_pool);
  const uint16_t* vp = static_cast<const uint16_t*>(v_pool);
#define KVS_ATTN(GG)                                                                                \
  hipLaunchKernelGGL(attn_split_kernel<GG>, grid, block, 0, s, P, qq, kp, vp, table, max_blocks, \
                     seq_lens, sel, sel_count, A.tps, A.n_splits, part_o, part_ml)
  switch (P.g) {
    case 1: KVS_ATTN(1); break;
    case 2: KVS_ATTN(2); break;
    case 4: KVS_ATTN(4); break;
    default: KVS_ATTN(8); break;
  }
#undef KVS_ATTN
  hipLaunchKernelGGL(attn_merge_kernel, dim3(P.Hq, batch), dim3(kDim), 0, s, P, seq_lens, sel_count,
                     A.tps, A.n_splits, part_o, part_ml, out);
  return hipGetLastError();
}

}  // namespace kvs
