// Top-k block selection for one (sequence, selection group) by one workgroup of NT lanes
// (used by kvs_topk_blocks and kvs_decode_step).
// KTransformers long-context sparse attention (lmnt.cn): §3.1 select the top-k blocks by score;
// §4.5 second_block_count.  Ties go to the lower block index; the output is in ascending order.
//
// Scores become order-preserving 32-bit keys (+0 and -0 share one key).  Finding the k-th largest key
// T, and how many keys equal to T are still needed, takes two stages:
//   1. value bins: kBins bins spread linearly over [min, max] of the candidate scores.  The bin index
//      is a monotone function of the score, so a bin above the boundary bin holds only keys above T.
//      A histogram (about n/kBins keys per bin, so LDS atomics rarely collide) and a suffix scan find
//      the bin that holds the k-th largest key.
//   2. inside that bin: up to 64 keys are gathered in LDS and wave 0 ranks them by counting (no
//      barriers); a crowded bin (many equal scores) goes through an MSB-first radix select (4 passes
//      of 8 bits).
// Each wave then walks its indices in ascending order 64 at a time, keeping every key > T and the
// lowest-indexed keys == T; ballots and popcounts give each kept block its slot, so the selection
// comes out in ascending block order.
//
// Rows of up to NT * KMAX blocks (every size the decode configurations use) keep their keys in
// registers: the score row, the table row and the sequence length are loaded together, and the
// candidate range is applied once the length has arrived.  Longer rows re-read their scores from
// memory on every pass.
#pragma once

#include "kvs_device.h"

namespace kvs {

__device__ inline uint32_t order_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if (f == 0.f) u = 0u;  // one key for +0 and -0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline float key_value(uint32_t u) {
  return __builtin_bit_cast(float, (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// A pointer every lane holds the same copy of, made visibly uniform (kept in scalar registers).
template <typename T>
__device__ inline T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

constexpr int kBins = 1024;     // value bins of stage 1
constexpr int kSubMax = 1024;   // keys of the boundary bin gathered in LDS for stage 2

// LDS the selection needs besides the staged keys.
struct TopkLds {
  int hist[kBins];
  uint32_t sub[kSubMax];
  int bcast[4];
  int wgt[16], weq[16];
  float fmin[16], fmax[16];
};

// Radix select of the `rem`-th largest among key(i), i < n.  Returns T; `rem` becomes the number of
// keys equal to T still to take.
template <int NT, typename KeyFn>
__device__ inline uint32_t radix_select(KeyFn key, int n, int& rem, TopkLds& S) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) S.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const uint32_t u = key(i);
      if ((u & pmask) == prefix) atomicAdd(&S.hist[(u >> shift) & 255], 1);
    }
    __syncthreads();
    if (tid < 64) {  // lane l owns digits 4l..4l+3; suffix sums from the high digits
      const int c0 = S.hist[4 * tid], c1 = S.hist[4 * tid + 1], c2 = S.hist[4 * tid + 2],
                c3 = S.hist[4 * tid + 3];
      const int own = c0 + c1 + c2 + c3;
      int suf = own;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_down(suf, d, 64);
        if (tid + d < 64) suf += y;
      }
      const int above_lane = suf - own;  // keys whose digit is above 4*tid+3
      if (above_lane < rem && suf >= rem) {
        int digit, above = above_lane;
        if (above + c3 >= rem) digit = 4 * tid + 3;
        else if ((above += c3) + c2 >= rem) digit = 4 * tid + 2;
        else if ((above += c2) + c1 >= rem) digit = 4 * tid + 1;
        else { above += c1; digit = 4 * tid; }
        S.bcast[0] = digit;
        S.bcast[1] = above;
      }
    }
    __syncthreads();
    rem -= S.bcast[1];
    prefix |= (uint32_t)S.bcast[0] << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  return prefix;
}

// Selects the top k of the n candidate scores row[0..n) (candidate i is logical block cand_lo + i),
// reading the scores again on every pass.  Writes sel[0..k) ascending; if tiles != nullptr also
// tiles[i] = trow[sel[i]] (physical ids).
template <int NT>
__device__ __attribute__((noinline)) void topk_select(const float* row, int n, int k, int cand_lo,
                                                      TopkLds& S, int32_t* sel, const int32_t* trow,
                                                      int32_t* tiles) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  row = uniform_ptr(row);
  sel = uniform_ptr(sel);
  trow = uniform_ptr(trow);
  tiles = uniform_ptr(tiles);
  n = __builtin_amdgcn_readfirstlane(n);
  k = __builtin_amdgcn_readfirstlane(k);
  cand_lo = __builtin_amdgcn_readfirstlane(cand_lo);
  auto put = [&](int32_t* p, int32_t v) { *p = v; };
  auto score = [&](int i) -> float { return row[i]; };
  if (k <= 0) return;
  if (k >= n) {
    for (int i = tid; i < n; i += NT) {
      put(sel + i, cand_lo + i);
      if (tiles) put(tiles + i, trow[cand_lo + i]);
    }
    return;
  }
  auto key = [&](int i) -> uint32_t { return order_key(score(i)); };

  // ---- stage 1: value bins over [min, max] ----
  float lo = INFINITY, hi = -INFINITY;
  for (int i = tid; i < n; i += NT) {
    const float v = key_value(key(i));
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    lo = fminf(lo, __shfl_xor(lo, m, 64));
    hi = fmaxf(hi, __shfl_xor(hi, m, 64));
  }
  if (lane == 0) { S.fmin[wv] = lo; S.fmax[wv] = hi; }
  for (int i = tid; i < kBins; i += NT) S.hist[i] = 0;
  __syncthreads();
  lo = S.fmin[0];
  hi = S.fmax[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) { lo = fminf(lo, S.fmin[w]); hi = fmaxf(hi, S.fmax[w]); }
  const float span = hi - lo;
  const float scale = span > 0.f && span < INFINITY ? (float)kBins / span : 0.f;
  auto bin_of = [&](uint32_t u) -> int {
    const float x = (key_value(u) - lo) * scale;  // monotone in the score
    return x >= (float)(kBins - 1) ? kBins - 1 : (int)x;
  };
  for (int i = tid; i < n; i += NT) atomicAdd(&S.hist[bin_of(key(i))], 1);
  __syncthreads();
  if (tid < 64) {  // boundary bin: lane l sums bins 16l..16l+15, suffix scan across lanes
    int own = 0;
#pragma unroll
    for (int b = 0; b < 16; ++b) own += S.hist[16 * tid + b];
    int suf = own;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_down(suf, d, 64);
      if (tid + d < 64) suf += y;
    }
    int above = suf - own;
    if (above < k && suf >= k) {
      int b = 16 * tid + 15;
      for (; b > 16 * tid; --b) {
        if (above + S.hist[b] >= k) break;
        above += S.hist[b];
      }
      S.bcast[0] = b;          // boundary bin
      S.bcast[1] = above;      // keys in higher bins (all selected)
      S.bcast[2] = 0;          // gather cursor of stage 2
      S.bcast[3] = S.hist[b];  // keys in the boundary bin (hist is reused below)
    }
  }
  __syncthreads();
  const int bstar = S.bcast[0];
  int rem = k - S.bcast[1];  // keys still to take from the boundary bin
  const int m_sub = S.bcast[3];

  // ---- stage 2: exact k-th key inside the boundary bin ----
  uint32_t T;
  if (m_sub <= kSubMax) {
    for (int i = tid; i < n; i += NT) {
      const uint32_t u = key(i);
      if (bin_of(u) == bstar) S.sub[atomicAdd(&S.bcast[2], 1)] = u;
    }
    __syncthreads();
    if (m_sub <= 64) {  // wave 0 ranks the few keys by counting
      if (tid < 64) {
        const uint32_t u = lane < m_sub ? S.sub[lane] : 0u;
        int gt = 0, ge = 0;
        for (int x = 0; x < m_sub; ++x) {
          const uint32_t v = S.sub[x];
          gt += v > u;
          ge += v >= u;
        }
        const bool is_t = lane < m_sub && gt < rem && ge >= rem;
        const unsigned long long bm = __ballot(is_t);
        const int src = __ffsll((long long)bm) - 1;  // some lane holds T (all such lanes agree)
        const uint32_t t = __shfl(u, src, 64);
        const int above_t = __shfl(gt, src, 64);
        if (lane == 0) { S.bcast[2] = (int)t; S.bcast[3] = rem - above_t; }
      }
      __syncthreads();
      T = (uint32_t)S.bcast[2];
      rem = S.bcast[3];
    } else {
      T = radix_select<NT>([&](int i) { return S.sub[i]; }, m_sub, rem, S);
    }
  } else {  // a crowded bin: select over all keys of that bin in place
    T = radix_select<NT>([&](int i) { const uint32_t u = key(i); return bin_of(u) == bstar ? u : 0u; },
                         n, rem, S);
  }
  // T is the k-th largest key; `rem` of the keys equal to T are taken

  // ---- ordered output: wave wv owns the contiguous index segment [s0, s1) ----
  const unsigned long long lt = (1ull << lane) - 1ull;
  const int seg = (n + NW - 1) / NW;
  const int s0 = min(n, wv * seg), s1 = min(n, s0 + seg);
  int n_gt = 0, n_eq = 0;
  for (int base = s0; base < s1; base += 64) {
    const int i = base + lane;
    const uint32_t u = i < s1 ? key(i) : 0u;
    n_gt += __popcll(__ballot(i < s1 && u > T));
    n_eq += __popcll(__ballot(i < s1 && u == T));
  }
  if (lane == 0) { S.wgt[wv] = n_gt; S.weq[wv] = n_eq; }
  __syncthreads();
  int eq_before = 0, pos = 0;
  for (int v = 0; v < wv; ++v) {
    pos += S.wgt[v] + max(0, min(S.weq[v], rem - eq_before));
    eq_before += S.weq[v];
  }
  for (int base = s0; base < s1; base += 64) {
    const int i = base + lane;
    const bool in = i < s1;
    const uint32_t u = in ? key(i) : 0u;
    const unsigned long long eqm = __ballot(in && u == T);
    const bool keep = in && (u > T || (u == T && eq_before + __popcll(eqm & lt) < rem));
    const unsigned long long km = __ballot(keep);
    if (keep) {
      const int slot = pos + __popcll(km & lt);
      put(sel + slot, cand_lo + i);
      if (tiles) put(tiles + slot, trow[cand_lo + i]);
    }
    pos += __popcll(km);
    eq_before += __popcll(eqm);
  }
}

// Register-resident selection of one (sequence, group) whose score row row[0..m) fits NT * KPT keys:
// lane l of wave w holds indices w*64*KPT + 64*c + l (c < KPT).  The row, the table row (trow,
// nullable) and *len are loaded together; candidates are the indices in [cand_lo, cand_hi) of the
// length's regions.  Writes *cnt = k_eff, sel[0..k_eff) ascending (and tiles[] = their physical ids
// when trow != nullptr), -1 in sel / tiles [k_eff, topk).  COH: the scores were stored by another
// workgroup of the same kernel (st_coh) and are read with coherent loads.
template <int NT, int KPT, bool COH = false>
__device__ __forceinline__ void topk_group_reg(const float* row, int m, const int32_t* len,
                                                         int initial_len, int local_len, int topk,
                                                         TopkLds& S, int32_t* sel, int32_t* cnt,
                                                         const int32_t* trow, int32_t* tiles) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  row = uniform_ptr(row);
  len = uniform_ptr(len);
  sel = uniform_ptr(sel);
  cnt = uniform_ptr(cnt);
  trow = uniform_ptr(trow);
  tiles = uniform_ptr(tiles);
  m = __builtin_amdgcn_readfirstlane(m);
  const int ibase = wv * 64 * KPT + lane;
  float v[KPT];
  int32_t ph[KPT];
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    const int i = ibase + 64 * c;
    const int ic = i < m ? i : 0;
    if constexpr (COH) v[c] = ld_coh_f1(coh_rsrc(row), ic * 4); else v[c] = row[ic];
    ph[c] = trow ? trow[ic] : 0;
  }
  const Regions rg = regions_of(*len, initial_len, local_len);
  const int lo = rg.cand_lo, hi = min(rg.cand_hi, m);
  const int n = max(0, hi - lo);
  const int k = min(topk, n);
  if (tid == 0) *cnt = k;
  for (int i = k + tid; i < topk; i += NT) {
    sel[i] = -1;
    if (trow) tiles[i] = -1;
  }
  if (k <= 0) return;
  auto ok = [&](int c) { const int i = ibase + 64 * c; return i >= lo && i < hi; };
  auto emit = [&](int slot, int c) {
    sel[slot] = ibase + 64 * c;
    if (trow) tiles[slot] = ph[c];
  };
  if (k >= n) {  // every candidate
#pragma unroll
    for (int c = 0; c < KPT; ++c)
      if (ok(c)) emit(ibase + 64 * c - lo, c);
    return;
  }
  uint32_t key[KPT];
  uint32_t kl = 0xFFFFFFFFu, kh = 0u;  // smallest / largest valid key of the lane (keys order as scores)
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    key[c] = ok(c) ? order_key(v[c]) : 0u;  // 0 is below every real key
    if (ok(c)) { kl = min(kl, key[c]); kh = max(kh, key[c]); }
  }
  kl = wave_min_u32(kl);
  kh = wave_max_u32(kh);
  if (lane == 0) {  // a wave without candidates reports an empty range
    S.fmin[wv] = kh ? key_value(kl) : INFINITY;
    S.fmax[wv] = kh ? key_value(kh) : -INFINITY;
  }
  for (int i = tid; i < kBins; i += NT) S.hist[i] = 0;
  __syncthreads();
  float fl = S.fmin[0], fh = S.fmax[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) { fl = fminf(fl, S.fmin[w]); fh = fmaxf(fh, S.fmax[w]); }
  const float span = fh - fl;
  const float scale = span > 0.f && span < INFINITY ? (float)kBins / span : 0.f;
  auto bin_of = [&](uint32_t u) -> int {
    const float x = (key_value(u) - fl) * scale;  // monotone in the score
    return x >= (float)(kBins - 1) ? kBins - 1 : (int)x;
  };
#pragma unroll
  for (int c = 0; c < KPT; ++c)
    if (ok(c)) atomicAdd(&S.hist[bin_of(key[c])], 1);
  __syncthreads();
  if (tid < 64) {  // boundary bin: lane l holds bins 16l..16l+15 in registers, suffix scan across lanes
    int hb[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int4 v4 = *reinterpret_cast<const int4*>(&S.hist[16 * tid + 4 * q]);
      hb[4 * q] = v4.x; hb[4 * q + 1] = v4.y; hb[4 * q + 2] = v4.z; hb[4 * q + 3] = v4.w;
    }
    int own = 0;
#pragma unroll
    for (int b = 0; b < 16; ++b) own += hb[b];
    int suf = own;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_down(suf, d, 64);
      if (tid + d < 64) suf += y;
    }
    if (suf - own < k && suf >= k) {  // the boundary bin is one of this lane's
      int above = suf - own, b = 15, cnt = hb[15];
#pragma unroll
      for (int bb = 15; bb >= 1; --bb) {  // highest bb with above + count(bins > bb) + hb[bb] >= k
        if (b == bb && above + hb[bb] < k) { above += hb[bb]; b = bb - 1; cnt = hb[bb - 1]; }
      }
      S.bcast[0] = 16 * tid + b;  // boundary bin
      S.bcast[1] = above;         // keys in higher bins (all selected)
      S.bcast[2] = 0;             // gather cursor
      S.bcast[3] = cnt;           // keys in the boundary bin (hist is reused below)
    }
  }
  __syncthreads();
  const int bstar = __builtin_amdgcn_readfirstlane(S.bcast[0]);
  int rem = k - __builtin_amdgcn_readfirstlane(S.bcast[1]);
  const int m_sub = __builtin_amdgcn_readfirstlane(S.bcast[3]);
  uint32_t T;
  if (m_sub <= 64) {  // gather the boundary bin, wave 0 ranks it by counting
#pragma unroll
    for (int c = 0; c < KPT; ++c)
      if (ok(c) && bin_of(key[c]) == bstar) S.sub[atomicAdd(&S.bcast[2], 1)] = key[c];
    __syncthreads();
    if (tid < 64) {  // rank by counting, the other keys broadcast from their lanes
      const uint32_t u = lane < m_sub ? S.sub[lane] : 0u;
      int gt = 0, ge = 0;
      for (int x = 0; x < m_sub; ++x) {
        const uint32_t w2 = (uint32_t)__builtin_amdgcn_readlane((int)u, x);
        gt += w2 > u;
        ge += w2 >= u;
      }
      const bool is_t = lane < m_sub && gt < rem && ge >= rem;
      const unsigned long long bm = __ballot(is_t);
      const int src = __ffsll((long long)bm) - 1;  // some lane holds T (all such lanes agree)
      const uint32_t t = __shfl(u, src, 64);
      const int above_t = __shfl(gt, src, 64);
      if (lane == 0) { S.bcast[2] = (int)t; S.bcast[3] = rem - above_t; }
    }
    __syncthreads();
    T = (uint32_t)S.bcast[2];
    rem = S.bcast[3];
  } else {  // a crowded bin (many equal scores): MSB-first radix select over that bin's keys
    uint32_t prefix = 0, pmask = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += NT) S.hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int c = 0; c < KPT; ++c) {
        const uint32_t u = key[c];
        if (ok(c) && bin_of(u) == bstar && (u & pmask) == prefix) atomicAdd(&S.hist[(u >> shift) & 255], 1);
      }
      __syncthreads();
      if (tid < 64) {  // lane l owns digits 4l..4l+3; suffix sums from the high digits
        const int c0 = S.hist[4 * tid], c1 = S.hist[4 * tid + 1], c2 = S.hist[4 * tid + 2],
                  c3 = S.hist[4 * tid + 3];
        const int own = c0 + c1 + c2 + c3;
        int suf = own;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int y = __shfl_down(suf, d, 64);
          if (tid + d < 64) suf += y;
        }
        const int above_lane = suf - own;
        if (above_lane < rem && suf >= rem) {
          int digit, above = above_lane;
          if (above + c3 >= rem) digit = 4 * tid + 3;
          else if ((above += c3) + c2 >= rem) digit = 4 * tid + 2;
          else if ((above += c2) + c1 >= rem) digit = 4 * tid + 1;
          else { above += c1; digit = 4 * tid; }
          S.bcast[0] = digit;
          S.bcast[1] = above;
        }
      }
      __syncthreads();
      rem -= S.bcast[1];
      prefix |= (uint32_t)S.bcast[0] << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
    T = prefix;
  }
  // T is the k-th largest key; `rem` of the keys equal to T are taken.  Ordered output:
  const unsigned long long lt = (1ull << lane) - 1ull;
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    n_gt += __popcll(__ballot(ok(c) && key[c] > T));
    n_eq += __popcll(__ballot(ok(c) && key[c] == T));
  }
  if (lane == 0) { S.wgt[wv] = n_gt; S.weq[wv] = n_eq; }
  __syncthreads();
  // keys > T and keys == T of the waves before this one (vector LDS reads, sums in registers); the
  // T-keys are taken in index order, so min(eq_before, rem) of them precede this wave's
  int gt_before = 0, eq_before = 0;
#pragma unroll
  for (int q = 0; q < NW / 4; ++q) {
    const int4 g4 = *reinterpret_cast<const int4*>(&S.wgt[4 * q]);
    const int4 e4 = *reinterpret_cast<const int4*>(&S.weq[4 * q]);
    gt_before += (4 * q < wv ? g4.x : 0) + (4 * q + 1 < wv ? g4.y : 0) + (4 * q + 2 < wv ? g4.z : 0) +
                 (4 * q + 3 < wv ? g4.w : 0);
    eq_before += (4 * q < wv ? e4.x : 0) + (4 * q + 1 < wv ? e4.y : 0) + (4 * q + 2 < wv ? e4.z : 0) +
                 (4 * q + 3 < wv ? e4.w : 0);
  }
  int pos = gt_before + min(eq_before, rem);
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    const unsigned long long eqm = __ballot(ok(c) && key[c] == T);
    const bool keep = ok(c) && (key[c] > T || (key[c] == T && eq_before + __popcll(eqm & lt) < rem));
    const unsigned long long km = __ballot(keep);
    if (keep) emit(pos + __popcll(km & lt), c);
    pos += __popcll(km);
    eq_before += __popcll(eqm);
  }
}

// The selection of group grp of sequence seq from the scores [batch][G][max_blocks]: sel (and, with a
// table and tiles, the physical ids in tiles) [batch][G][topk] ascending and -1 padded,
// sel_count [batch][G].  Rows of up to NT * KMAX blocks stay in registers.  COH (rows of up to
// NT * KMAX blocks only): the scores come from another workgroup of the same kernel.
template <int NT, int KMAX, bool COH = false>
__device__ inline void topk_group(const Params& P, const float* __restrict__ scores,
                                  const int32_t* __restrict__ seq_lens, int max_blocks,
                                  int32_t* __restrict__ sel, int32_t* __restrict__ sel_count,
                                  const int32_t* __restrict__ table, int32_t* __restrict__ tiles,
                                  int seq, int grp, TopkLds& S) {
  const size_t row = (size_t)seq * P.G + grp;
  const float* srow = scores + row * max_blocks;
  int32_t* out = sel + row * P.topk;
  int32_t* tout = tiles ? tiles + row * P.topk : nullptr;
  const int32_t* trow = tiles && table ? table + (size_t)seq * max_blocks : nullptr;
  const int32_t* len = seq_lens + seq;
#define KVS_TOPK_REG(KPT)                                                                            \
  topk_group_reg<NT, KPT, COH>(srow, max_blocks, len, P.initial_len, P.local_len, P.topk, S, out,         \
                          sel_count + row, trow, tout)
  if (max_blocks <= NT * 4) { KVS_TOPK_REG(4); return; }
  if (KMAX >= 8 && max_blocks <= NT * 8) { KVS_TOPK_REG(8); return; }
  if (KMAX >= 16 && max_blocks <= NT * 16) { KVS_TOPK_REG(16); return; }
  if (KMAX >= 32 && max_blocks <= NT * 32) { KVS_TOPK_REG(32); return; }
#undef KVS_TOPK_REG
  if constexpr (COH) return;  // not reached: callers keep coherent rows within NT * KMAX blocks
  const int tid = threadIdx.x;
  const Regions rg = regions_of(*len, P.initial_len, P.local_len);
  const int n = max(0, min(rg.cand_hi, max_blocks) - rg.cand_lo);
  const int k = min(P.topk, n);
  if (tid == 0) sel_count[row] = k;
  for (int i = k + tid; i < P.topk; i += NT) {
    out[i] = -1;
    if (trow) tout[i] = -1;
  }
  topk_select<NT>(srow + rg.cand_lo, n, k, rg.cand_lo, S, out, trow, trow ? tout : nullptr);
}

}  // namespace kvs
