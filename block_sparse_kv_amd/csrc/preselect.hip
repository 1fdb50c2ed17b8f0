// Preselect (KTransformers long-context article §4.4, after SnapKV; §4.5 preselect_block_count):
// before decoding, a set of blocks is chosen from the attention the question's tokens pay the
// context, and every later selection is confined to it.
//  * block_score_kernel: a block's preselect score is the sum of its tokens' scores
//    (kvs_token_importance), -inf outside the candidates -- the layout of the block scores, so the
//    set is the ordinary top-k of these rows.
//  * block_pool_score_kernel: the pooled form of the article's preselect pseudocode (§4.6
//    preselect_block: pool1d over the window's votes, then the best tokens and their blocks).  A
//    token's pooled vote is the mean of the Context votes in a centred window of pool_kernel
//    tokens, zero outside the Context; taking tokens in descending pooled vote until enough
//    distinct blocks are hit ranks each block by its best pooled token, which is the score stored.
//  * The confined decode step scores every candidate as usual.  For sets of up to 256 blocks one
//    workgroup per (sequence, group) ranks the set's current candidates by counting
//    (presel_select_kernel).  For larger sets compact_kernel keeps, per
//    (sequence, group), the scores of the set's blocks that are still candidates, in block order,
//    as one row of a compacted batch (each row its own "sequence" of n_eff blocks with no Initial or
//    Local part), the ordinary top-k selects in it, and map_back_kernel turns the picks into block
//    ids for the attention tiles and the merge.
#include "kvs_launch.h"

namespace kvs {

// One wave per (candidate block, group, sequence): sum of the block's 128 token scores.
__global__ __launch_bounds__(256) void block_score_kernel(Params P, const float* __restrict__ imp,
                                                          const int32_t* __restrict__ seq_lens,
                                                          int max_blocks, float* __restrict__ bs) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6), gr = blockIdx.y, seq = blockIdx.z;
  const int lane = threadIdx.x & 63;
  if (b >= max_blocks) return;
  const Regions rg = regions_of(seq_lens[seq], P.initial_len, P.local_len);
  const size_t row = (size_t)seq * P.G + gr;
  float s = 0.f;
  if (b >= rg.cand_lo && b < rg.cand_hi) {
    const float2 x = reinterpret_cast<const float2*>(imp + row * (size_t)max_blocks * kBlock + (size_t)b * kBlock)[lane];
    s = wave_sum_f32(x.x + x.y);
  } else {
    s = -INFINITY;
  }
  if (lane == 0) bs[row * max_blocks + b] = s;
}

// One wave per (candidate block, group, sequence): the largest pooled vote among the block's 128
// tokens, divided by pool_kernel.  The wave stages the votes of tokens b*128-64 .. b*128+191 (zero
// outside the Context [cand_lo*128, cand_hi*128)) in LDS; lane l sums the windows of tokens l and
// l+64 in ascending token order.  pool_kernel is odd and <= 127, so every window stays in the
// staged span.
__global__ __launch_bounds__(256) void block_pool_score_kernel(Params P, const float* __restrict__ imp,
                                                               const int32_t* __restrict__ seq_lens,
                                                               int max_blocks, int pool_kernel,
                                                               float* __restrict__ bs) {
  __shared__ float4 stage[4][64];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = blockIdx.x * 4 + w, gr = blockIdx.y, seq = blockIdx.z;
  const Regions rg = regions_of(seq_lens[seq], P.initial_len, P.local_len);
  const size_t row = (size_t)seq * P.G + gr;
  const int lo = rg.cand_lo * kBlock, hi = rg.cand_hi * kBlock, n_tok = max_blocks * kBlock;
  // votes of tokens p .. p+3, loaded from a clamped in-row position and masked to the Context
  const int p = b * kBlock - 64 + 4 * lane;
  const int pc = min(max(p, 0), n_tok - 4);
  const float4 x = reinterpret_cast<const float4*>(imp + row * (size_t)n_tok)[pc >> 2];
  float4 v;
  v.x = (p >= lo && p < hi) ? x.x : 0.f;
  v.y = (p + 1 >= lo && p + 1 < hi) ? x.y : 0.f;
  v.z = (p + 2 >= lo && p + 2 < hi) ? x.z : 0.f;
  v.w = (p + 3 >= lo && p + 3 < hi) ? x.w : 0.f;
  stage[w][lane] = v;
  __syncthreads();
  const float* st = reinterpret_cast<const float*>(stage[w]);
  const int h = pool_kernel >> 1;
  float best = -INFINITY;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int i = lane + 64 * half;  // token b*128 + i sits at st[64 + i]
    float acc = 0.f;
    for (int u = 64 + i - h; u <= 64 + i + h; ++u) acc += st[u];
    best = fmaxf(best, acc);
  }
  best = wave_max_f32(best);
  if (lane == 0 && b < max_blocks)
    bs[row * max_blocks + b] = (b >= rg.cand_lo && b < rg.cand_hi) ? best / (float)pool_kernel : -INFINITY;
}

// One wave per (group, sequence) row: the set's blocks that are current candidates, in order (a
// ballot prefix places each kept entry).  cs / cid: [batch * G][n_presel] compacted scores and their
// block ids, -inf / -1 padded; clen: the row's length in tokens (n_eff * 128) for the top-k over the
// compacted rows.
__global__ __launch_bounds__(256) void compact_kernel(Params P, const float* __restrict__ scores, int max_blocks,
                                                      const int32_t* __restrict__ seq_lens,
                                                      const int32_t* __restrict__ presel, int n_presel,
                                                      int rows, float* __restrict__ cs, int32_t* __restrict__ cid,
                                                      int32_t* __restrict__ clen) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int seq = row / P.G;
  const Regions rg = regions_of(seq_lens[seq], P.initial_len, P.local_len);
  const int32_t* ps = presel + (size_t)row * n_presel;
  float* o = cs + (size_t)row * n_presel;
  int32_t* oi = cid + (size_t)row * n_presel;
  const unsigned long long lt = (1ull << lane) - 1ull;
  int n = 0;
  for (int i0 = 0; i0 < n_presel; i0 += 64) {
    const int i = i0 + lane;
    const int b = i < n_presel ? ps[i] : -1;
    const bool ok = b >= rg.cand_lo && b < rg.cand_hi && b < max_blocks;
    const unsigned long long m = __ballot(ok);
    if (ok) {
      const int at = n + __popcll(m & lt);
      o[at] = scores[(size_t)row * max_blocks + b];
      oi[at] = b;
    }
    n += __popcll(m);
  }
  for (int i = n + lane; i < n_presel; i += 64) {
    o[i] = -INFINITY;
    oi[i] = -1;
  }
  if (lane == 0) clen[row] = n * kBlock;
}

// One thread per (row, pick): compacted index -> block id; -1 stays -1.
__global__ __launch_bounds__(256) void map_back_kernel(const int32_t* __restrict__ csel, int topk,
                                                       const int32_t* __restrict__ cid, int n_presel, int total,
                                                       int32_t* __restrict__ sel) {
  const int x = blockIdx.x * 256 + threadIdx.x;
  if (x >= total) return;
  const int row = x / topk, j = csel[x];
  sel[x] = j >= 0 && j < n_presel ? cid[(size_t)row * n_presel + j] : -1;
}

// Sets of up to 256 blocks: the whole confined selection of one (sequence, group) row in one
// workgroup of 1024 lanes.  Entry i's rank among the set's current candidates (higher score, or equal
// and lower block, beats it) is counted by four lanes, one per quarter of the entries, with 16-byte
// LDS reads; the k_eff best are kept and a prefix over the (ascending) set gives each its slot.
constexpr int kPreselFused = 256;

__global__ __launch_bounds__(1024) void presel_select_kernel(Params P, const float* __restrict__ scores,
                                                             int max_blocks, const int32_t* __restrict__ seq_lens,
                                                             const int32_t* __restrict__ presel, int n_presel,
                                                             int32_t* __restrict__ sel,
                                                             int32_t* __restrict__ sel_count) {
  __shared__ __attribute__((aligned(16))) float ss[kPreselFused];
  __shared__ __attribute__((aligned(16))) int sb[kPreselFused];
  __shared__ int part[4][kPreselFused];
  __shared__ int wcnt[kPreselFused / 64];
  const int row = blockIdx.x, tid = threadIdx.x, e = tid & (kPreselFused - 1), q = tid >> 8;
  const Regions rg = regions_of(seq_lens[row / P.G], P.initial_len, P.local_len);
  int b = -1;
  bool ok = false;
  float v = 0.f;
  if (q == 0) {
    b = e < n_presel ? presel[(size_t)row * n_presel + e] : -1;
    ok = b >= rg.cand_lo && b < rg.cand_hi && b < max_blocks;
    v = ok ? scores[(size_t)row * max_blocks + b] : 0.f;
    ss[e] = v;
    sb[e] = ok ? b : -1;
  }
  const int n_ok = __syncthreads_count(ok);
  const int k = min(P.topk, n_ok);
  {
    const float vi = ss[e];
    const int bi = sb[e];
    int r = 0;
#pragma unroll 4
    for (int j = 64 * q; j < 64 * q + 64; j += 4) {
      const float4 v4 = *reinterpret_cast<const float4*>(&ss[j]);
      const int4 b4 = *reinterpret_cast<const int4*>(&sb[j]);
      r += b4.x >= 0 && (v4.x > vi || (v4.x == vi && b4.x < bi));
      r += b4.y >= 0 && (v4.y > vi || (v4.y == vi && b4.y < bi));
      r += b4.z >= 0 && (v4.z > vi || (v4.z == vi && b4.z < bi));
      r += b4.w >= 0 && (v4.w > vi || (v4.w == vi && b4.w < bi));
    }
    part[q][e] = r;
  }
  __syncthreads();  // partial ranks
  const int lane = tid & 63, w = tid >> 6;  // waves 0..3 hold the entries (q == 0)
  bool take = false;
  unsigned long long m = 0ull;
  if (q == 0) {
    take = ok && part[0][e] + part[1][e] + part[2][e] + part[3][e] < k;
    m = __ballot(take);
    if (lane == 0) wcnt[w] = __popcll(m);
  }
  __syncthreads();  // every wave, the idle ones included
  if (q == 0) {
    int slot = __popcll(m & ((1ull << lane) - 1ull));
    for (int x = 0; x < w; ++x) slot += wcnt[x];
    int32_t* out = sel + (size_t)row * P.topk;
    if (take) out[slot] = b;
    for (int i = k + tid; i < P.topk; i += kPreselFused) out[i] = -1;
    if (tid == 0) sel_count[row] = k;
  }
}

hipError_t launch_presel_select(const Params& P, const float* scores, int max_blocks, const int32_t* seq_lens,
                                const int32_t* presel, int n_presel, int batch, int32_t* sel,
                                int32_t* sel_count, hipStream_t s) {
  hipLaunchKernelGGL(presel_select_kernel, dim3(batch * P.G), dim3(1024), 0, s, P, scores, max_blocks,
                     seq_lens, presel, n_presel, sel, sel_count);
  return hipGetLastError();
}

hipError_t launch_block_scores(const Params& P, const float* imp, const int32_t* seq_lens, int batch,
                               int max_blocks, int pool_kernel, float* bs, hipStream_t s) {
  const dim3 grid((max_blocks + 3) / 4, P.G, batch);
  if (pool_kernel > 0)
    hipLaunchKernelGGL(block_pool_score_kernel, grid, dim3(256), 0, s, P, imp, seq_lens, max_blocks,
                       pool_kernel, bs);
  else
    hipLaunchKernelGGL(block_score_kernel, grid, dim3(256), 0, s, P, imp, seq_lens, max_blocks, bs);
  return hipGetLastError();
}

hipError_t launch_compact(const Params& P, const float* scores, int max_blocks, const int32_t* seq_lens,
                          const int32_t* presel, int n_presel, int batch, float* cs, int32_t* cid,
                          int32_t* clen, hipStream_t s) {
  const int rows = batch * P.G;
  hipLaunchKernelGGL(compact_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, P, scores, max_blocks, seq_lens,
                     presel, n_presel, rows, cs, cid, clen);
  return hipGetLastError();
}

hipError_t launch_map_back(const int32_t* csel, int topk, const int32_t* cid, int n_presel, int rows,
                           int32_t* sel, hipStream_t s) {
  const int total = rows * topk;
  if (total > 0)
    hipLaunchKernelGGL(map_back_kernel, dim3((total + 255) / 256), dim3(256), 0, s, csel, topk, cid, n_presel,
                       total, sel);
  return hipGetLastError();
}

}  // namespace kvs
