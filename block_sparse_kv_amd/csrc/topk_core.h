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

constexpr int kBndMax = 64;     // register path: a boundary bin of up to kBndMax keys is ranked by one wave
constexpr int kBmapWords = 512; // register path: rows of up to 32 * kBmapWords blocks

// LDS of a selection.
struct TopkLds {
  alignas(16) int hist[kBins + 4];          // value bins; the register path counts non-candidates at [kBins]
  alignas(16) uint32_t sub[kSubMax];        // keys of the boundary bin (re-read path)
  alignas(16) unsigned long long bcomp[kBndMax];  // register path: boundary-bin keys, key << 32 | ~index
  alignas(16) uint32_t bmap[kBmapWords];    //   boundary-bin blocks taken, one bit per block
  alignas(16) int wgt[16], weq[16], woff[16];
  alignas(16) float fmin[16], fmax[16];
  int bcast[4];
  int cur;                                  // append cursor of bcomp
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
// tiles[i] = trow[sel[i]] (physical ids).  COH: the scores were stored by other workgroups of the same
// kernel (st_coh) and are read with coherent loads.
template <int NT, bool COH = false>
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
  const __amdgpu_buffer_rsrc_t rs = coh_rsrc(row);
  auto score = [&](int i) -> float {
    if constexpr (COH) return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, i * 4, 0, kSc1));
    else return row[i];
  };
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

// ---- register-resident selection ------------------------------------------------------------------
// Keys live in registers: lane l of wave w holds positions w*64*KPT + 64*c + l (c < KPT), so each wave
// owns a contiguous position range and ballots over its columns, in (column, lane) order, visit its
// positions in ascending order.
//
// topk_reg_take: the top k (1 <= k < number of candidates) of the candidate positions (bit c of okb
// set) by (value desc, position asc).  Each candidate's value bin stays in a register, so only the
// histogram goes through LDS.  Every wave reads the whole histogram and finds the boundary bin itself
// (DPP prefix sum; no barrier waits on one wave's search).  The keys of the bins above it are taken.
// When every key of the boundary bin is needed (the usual case: value bins are sparse near the k-th
// key) they are taken too; a boundary bin of at most kBndMax keys is otherwise gathered and ranked by
// (key, lower position first) in one wave, which marks the ones it takes in a bitmap; a crowded one
// goes through a radix select of the k-th key.  Returns the take bits of the lane's keys (bit c) and,
// in *off, the output slot of the wave's first taken key.
template <int NT, int KPT>
__device__ __forceinline__ uint32_t topk_reg_take(const float (&v)[KPT], uint32_t okb, int k, int ibase,
                                                  TopkLds& S, int* off_out) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  auto ok = [&](int c) { return ((okb >> c) & 1u) != 0u; };

  // ---- value range of the candidates ----
  float vl = INFINITY, vh = -INFINITY;
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    vl = fminf(vl, ok(c) ? v[c] : INFINITY);
    vh = fmaxf(vh, ok(c) ? v[c] : -INFINITY);
  }
  vl = wave_min_f32(vl);
  vh = wave_max_f32(vh);
  if (lane == 0) { S.fmin[wv] = vl; S.fmax[wv] = vh; }
  static_assert((kBins + 4) % 4 == 0, "the histogram clears in 16-byte stores");
  for (int i = tid; i < (kBins + 4) / 4; i += NT) reinterpret_cast<int4*>(S.hist)[i] = make_int4(0, 0, 0, 0);
  for (int i = tid; i < NT * KPT / 32; i += NT) S.bmap[i] = 0u;
  if (tid == 0) S.cur = 0;
  __syncthreads();
  float fl = S.fmin[0], fh = S.fmax[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) { fl = fminf(fl, S.fmin[w]); fh = fmaxf(fh, S.fmax[w]); }
  const float span = fh - fl;
  // bin(v) = min(v * scale - fl * scale, kBins - 1), truncated: monotone in v for any fixed scale >= 0
  // (a rounding just below 0 truncates to bin 0).  A range that is empty or not finite gives scale 0;
  // NaN scores land in the top bin.
  const float scale = span > 0.f && span < INFINITY ? (float)kBins * __builtin_amdgcn_rcpf(span) : 0.f;
  const float boff = -fl * scale;
  auto bin = [&](float x) { return (int)fminf(fmaf(x, scale, boff), (float)(kBins - 1)); };

  // ---- histogram: bin of a candidate in a register, -1 for the others (counted in hist[kBins]) ----
  int b[KPT];
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    b[c] = ok(c) ? bin(v[c]) : -1;
    atomicAdd(&S.hist[min((unsigned)b[c], (unsigned)kBins)], 1);
  }
  __syncthreads();

  // ---- boundary bin, in every wave.  Lane l sums bins [kBins - 16(l+1), kBins - 16l); a prefix sum
  // over lanes counts keys from the top and names the lane whose 16 bins hold the k-th key; then
  // lanes 0..15 take those bins, top bin first, and a prefix sum inside the row names the bin. ----
  int bstar, above, m_sub;
  {
    const int4* h4 = reinterpret_cast<const int4*>(&S.hist[kBins - 16 * (lane + 1)]);
    const int4 a0 = h4[0], a1 = h4[1], a2 = h4[2], a3 = h4[3];
    const int own = (a0.x + a0.y + a0.z + a0.w) + (a1.x + a1.y + a1.z + a1.w) +
                    (a2.x + a2.y + a2.z + a2.w) + (a3.x + a3.y + a3.z + a3.w);
    const int incl = wave_incl_scan(own);
    const unsigned long long bl = __ballot(incl - own < k && incl >= k);  // one lane: n > k keys
    const int src = __builtin_amdgcn_readfirstlane(__ffsll((long long)bl) - 1);
    const int above_src = __builtin_amdgcn_readlane(incl - own, src);
    const int top = kBins - 16 * src - 1;  // the highest of the src lane's bins
    const int hj = lane < 16 ? S.hist[top - lane] : 0;
    int cj = hj;  // inclusive prefix over lanes 0..15 of row 0
    cj += __builtin_amdgcn_update_dpp(0, cj, 0x111, 0xF, 0xF, true);  // row_shr:1
    cj += __builtin_amdgcn_update_dpp(0, cj, 0x112, 0xF, 0xF, true);  // row_shr:2
    cj += __builtin_amdgcn_update_dpp(0, cj, 0x114, 0xF, 0xF, true);  // row_shr:4
    cj += __builtin_amdgcn_update_dpp(0, cj, 0x118, 0xF, 0xF, true);  // row_shr:8
    const unsigned long long bj = __ballot(lane < 16 && above_src + cj - hj < k && above_src + cj >= k);
    const int jb = __builtin_amdgcn_readfirstlane(__ffsll((long long)bj) - 1);
    bstar = top - jb;
    above = above_src + __builtin_amdgcn_readlane(cj - hj, jb);
    m_sub = __builtin_amdgcn_readlane(hj, jb);
  }
  const int rem = k - above;  // keys still to take from the boundary bin, 1..m_sub
  const unsigned long long lt = (1ull << lane) - 1ull;
  uint32_t take = 0u;

  if (rem == m_sub) {
    // ---- the whole boundary bin is taken: the keys of bins >= bstar are the selection ----
    int n_ge = 0;
#pragma unroll
    for (int c = 0; c < KPT; ++c) {
      take |= (b[c] >= bstar ? 1u : 0u) << c;
      n_ge += __popcll(__ballot(b[c] >= bstar));
    }
    if (lane == 0) S.wgt[wv] = n_ge;
    __syncthreads();
    int off = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) off += w < wv ? S.wgt[w] : 0;
    *off_out = off;
    return take;
  }

  if (m_sub <= kBndMax) {
    // ---- keys of higher bins are all taken: each wave counts its own; the boundary bin's keys are
    // gathered for ranking.  The wave's boundary keys take one range of bcomp: a prefix sum over lanes
    // places each lane's keys, and one LDS atomic per wave places the wave. ----
    int n_above = 0, nb = 0;
#pragma unroll
    for (int c = 0; c < KPT; ++c) {
      n_above += __popcll(__ballot(b[c] > bstar));
      nb += b[c] == bstar;
    }
    const int nb_incl = wave_incl_scan(nb);
    const int nb_wave = __builtin_amdgcn_readlane(nb_incl, 63);
    if (nb_wave != 0) {
      int base = 0;
      if (lane == 0) base = atomicAdd(&S.cur, nb_wave);
      int at = __builtin_amdgcn_readlane(base, 0) + nb_incl - nb;
#pragma unroll
      for (int c = 0; c < KPT; ++c)
        if (b[c] == bstar)
          S.bcomp[at++] = ((unsigned long long)order_key(v[c]) << 32) | (uint32_t)~(uint32_t)(ibase + 64 * c);
    }
    if (lane == 0) S.wgt[wv] = n_above;
    __syncthreads();
    if (wv == 0) {
      // rank of each boundary key: how many beat it (higher key, or equal and lower position); the best
      // rem are taken and marked in the bitmap, and every wave gets its output offset
      const bool mine = lane < m_sub;
      const unsigned long long cj = S.bcomp[mine ? lane : 0];
      int r = 0;
#pragma unroll 4
      for (int x = 0; x < m_sub; x += 2) {
        const ulonglong2 c2 = *reinterpret_cast<const ulonglong2*>(&S.bcomp[x]);
        r += (c2.x > cj) + (x + 1 < m_sub && c2.y > cj);
      }
      const int wj = (int)(~(uint32_t)cj) / (64 * KPT);
      const bool tk = mine && r < rem;
      const int ij = (int)~(uint32_t)cj;
      if (tk) atomicOr(&S.bmap[ij >> 5], 1u << (ij & 31));
      int bsel = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int cw = __popcll(__ballot(tk && wj == w));
        bsel = lane == w ? cw : bsel;
      }
      const int tot = lane < NW ? S.wgt[lane] + bsel : 0;
      const int incl = wave_incl_scan(tot);
      if (lane < NW) S.woff[lane] = incl - tot;
    }
    __syncthreads();
    // Key ibase + 64c is bit (lane & 31) of bitmap word (ibase >> 5) + 2c: the words are read together.
    uint32_t wd[KPT];
#pragma unroll
    for (int c = 0; c < KPT; ++c) wd[c] = S.bmap[(ibase >> 5) + 2 * c];
#pragma unroll
    for (int c = 0; c < KPT; ++c)
      take |= (b[c] > bstar || (b[c] == bstar && ((wd[c] >> (lane & 31)) & 1u)) ? 1u : 0u) << c;
    *off_out = S.woff[wv];
    return take;
  }

  // ---- a crowded boundary bin: radix select of the k-th key inside the boundary bin ----
  auto key = [&](int c) { return order_key(v[c]); };  // recomputed: no register array for the rare case
  int remT = rem;
  uint32_t prefix = 0, pmask = 0;
  __syncthreads();  // every wave has read the value histogram
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) S.hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < KPT; ++c)
      if (b[c] == bstar && (key(c) & pmask) == prefix) atomicAdd(&S.hist[(key(c) >> shift) & 255], 1);
    __syncthreads();
    if (tid < 64) {  // lane l owns digits 4l..4l+3; suffix sums from the high digits
      const int c0 = S.hist[4 * tid], c1 = S.hist[4 * tid + 1], c2 = S.hist[4 * tid + 2],
                c3 = S.hist[4 * tid + 3];
      const int own = c0 + c1 + c2 + c3;
      int suf = own;
#pragma unroll
      for (int dd = 1; dd < 64; dd <<= 1) {
        const int y = __shfl_down(suf, dd, 64);
        if (tid + dd < 64) suf += y;
      }
      const int above_lane = suf - own;
      if (above_lane < remT && suf >= remT) {
        int digit, ab = above_lane;
        if (ab + c3 >= remT) digit = 4 * tid + 3;
        else if ((ab += c3) + c2 >= remT) digit = 4 * tid + 2;
        else if ((ab += c2) + c1 >= remT) digit = 4 * tid + 1;
        else { ab += c1; digit = 4 * tid; }
        S.bcast[0] = digit;
        S.bcast[1] = ab;
      }
    }
    __syncthreads();
    remT -= S.bcast[1];
    prefix |= (uint32_t)S.bcast[0] << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t T = prefix;  // the k-th largest key: keys of higher bins, keys > T of the boundary
                              // bin and the remT lowest-positioned keys == T are taken
  auto gt = [&](int c) { return b[c] > bstar || (b[c] == bstar && key(c) > T); };
  auto eq = [&](int c) { return b[c] == bstar && key(c) == T; };
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    n_gt += __popcll(__ballot(gt(c)));
    n_eq += __popcll(__ballot(eq(c)));
  }
  if (lane == 0) { S.wgt[wv] = n_gt; S.weq[wv] = n_eq; }
  __syncthreads();
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
  *off_out = gt_before + min(eq_before, remT);
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    const unsigned long long eqm = __ballot(eq(c));
    take |= (gt(c) || (eq(c) && eq_before + __popcll(eqm & lt) < remT) ? 1u : 0u) << c;
    eq_before += __popcll(eqm);
  }
  return take;
}

// Writes the taken keys in ascending position order from slot `off` of the wave on: sel[slot] = the
// key's id (its position, or idv[c]), tiles[slot] = ph[c] when with_tiles.
template <int KPT>
__device__ __forceinline__ void topk_reg_write(uint32_t take, int off, int k, int ibase, const int32_t (&idv)[KPT],
                                               bool use_ids, const int32_t (&ph)[KPT], bool with_tiles,
                                               __attribute__((address_space(1))) int32_t* sel,
                                               __attribute__((address_space(1))) int32_t* tiles) {
  const int lane = threadIdx.x & 63;
  const unsigned long long lt = (1ull << lane) - 1ull;
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    const bool t = (take >> c) & 1u;
    const unsigned long long km = __ballot(t);
    if (km != 0ull) {
      const int slot = off + __popcll(km & lt);
      if (t && slot < k) {
        sel[slot] = use_ids ? idv[c] : ibase + 64 * c;
        if (with_tiles) tiles[slot] = ph[c];
      }
      off += __popcll(km);
    }
  }
}

// Register-resident selection of one (sequence, group) whose score row row[0..m) fits NT * KPT keys.
// The row, the table row (trow, nullable) and *len are loaded together; candidates are the indices in
// [cand_lo, cand_hi) of the length's regions.  Writes *cnt = k_eff, sel[0..k_eff) ascending (and
// tiles[] = their physical ids when trow != nullptr), -1 in sel / tiles [k_eff, topk).  COH: the
// scores were stored by another workgroup of the same kernel (st_coh) and are read with coherent
// loads.  The count and the -1 padding are stored after the last barrier (a barrier waits for every
// store the wave has issued).
template <int NT, int KPT, bool COH = false>
__device__ __forceinline__ void topk_group_reg(const float* row, int m, const int32_t* len,
                                                int initial_len, int local_len, int topk,
                                                TopkLds& S, int32_t* sel_, int32_t* cnt_,
                                                const int32_t* trow, int32_t* tiles_) {
  static_assert(NT % 256 == 0 && NT <= 1024, "4 to 16 waves");
  static_assert(NT * KPT <= 32 * kBmapWords, "one bitmap bit per block");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  auto sel = gptr(sel_);
  auto cnt = gptr(cnt_);
  auto tiles = gptr(tiles_);
  const bool with_tiles = trow != nullptr;
  const int ibase = wv * 64 * KPT + lane;
  const __amdgpu_buffer_rsrc_t rs = span_rsrc(row, m * 4);
  const __amdgpu_buffer_rsrc_t rt = span_rsrc(trow, with_tiles ? m * 4 : 0);
  float v[KPT];
  int32_t ph[KPT];
#pragma unroll
  for (int c = 0; c < KPT; ++c)
    v[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (ibase + 64 * c) * 4, 0,
                                                                          COH ? kSc1 : 0));
#pragma unroll
  for (int c = 0; c < KPT; ++c) ph[c] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rt, (ibase + 64 * c) * 4, 0, 0);
  const Regions rg = regions_of(ld_uniform_i32(len), initial_len, local_len);
  const int lo = rg.cand_lo, hi = min(rg.cand_hi, m);
  const int n = max(0, hi - lo);
  const int k = min(topk, n);
  auto finish = [&]() {
    if (tid == 0) *cnt = k;
    for (int i = k + tid; i < topk; i += NT) {
      sel[i] = -1;
      if (with_tiles) tiles[i] = -1;
    }
  };
  if (k <= 0) { finish(); return; }
  const int d = ibase - lo;  // candidate offset of column 0
  uint32_t okb = 0u;
#pragma unroll
  for (int c = 0; c < KPT; ++c) okb |= ((unsigned)(d + 64 * c) < (unsigned)n ? 1u : 0u) << c;
  const int32_t none[KPT] = {};
  if (k >= n) {  // every candidate
    finish();
#pragma unroll
    for (int c = 0; c < KPT; ++c)
      if ((okb >> c) & 1u) {
        sel[d + 64 * c] = ibase + 64 * c;
        if (with_tiles) tiles[d + 64 * c] = ph[c];
      }
    return;
  }
  int off = 0;
  const uint32_t take = topk_reg_take<NT, KPT>(v, okb, k, ibase, S, &off);
  finish();
  topk_reg_write<KPT>(take, off, k, ibase, none, false, ph, with_tiles, sel, tiles);
}

// Walks the taken keys as topk_reg_write does (ascending position, slots from `off` of the wave on):
// the lane holding entry `slot` puts its id (idv) and physical id (ph) into slot_lds[0..1]; with
// `writer`, sel[j] = the id of entry j for every j < k.  Without branches per column: each column's
// ballot and the lane's count of lower taken lanes place its key, and one store hands the entry over.
template <int KPT>
__device__ __forceinline__ void topk_slot_walk(uint32_t take, int off, int k, const int32_t (&idv)[KPT],
                                               const int32_t (&ph)[KPT], int slot, int* slot_lds, bool writer,
                                               __attribute__((address_space(1))) int32_t* sel) {
  bool hit = false;
  int hid = 0, hph = 0;
  int o = off;
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    const bool t = (take >> c) & 1u;
    const unsigned long long km = __ballot(t);
    const int j = o + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(km >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)km, 0u));
    const bool h = t && j == slot;
    hid = h ? idv[c] : hid;
    hph = h ? ph[c] : hph;
    hit = hit || h;
    o += __popcll(km);
  }
  if (hit) { slot_lds[0] = hid; slot_lds[1] = hph; }
  if (writer) {
#pragma unroll
    for (int c = 0; c < KPT; ++c) {
      const bool t = (take >> c) & 1u;
      const unsigned long long km = __ballot(t);
      const int j = off + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(km >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)km, 0u));
      if (t && j < k) sel[j] = idv[c];
      off += __popcll(km);
    }
  }
}

// One entry of the selection of a (sequence, group), made by a workgroup that attends it: the same
// selection as topk_group_reg's over the score row row[0..m) (stored by an earlier launch), loaded with
// the table row and *len, keys in registers.  Returns entry `slot` of the ascending selection -- its
// logical block in .x and physical id (trow) in .y -- or (-1, -1) when slot >= k_eff.  slot_lds: two
// ints of the workgroup's LDS outside S, through which the entry's owner lane hands it over.  With
// `writer` the workgroup also writes the whole selection: *cnt = k_eff, sel[0..k_eff) ascending,
// -1 in [k_eff, topk).  tl_rec: the workgroup's timeline record (timeline build), or null.
template <int NT, int KPT>
__device__ __forceinline__ int2 topk_slot_reg(const float* row, int m, const int32_t* len, int initial_len,
                                              int local_len, int topk, int slot, TopkLds& S,
                                              const int32_t* trow, bool writer, int32_t* sel_,
                                              int32_t* cnt_, int* slot_lds, unsigned long long* tl_rec) {
  static_assert(NT % 256 == 0 && NT <= 1024, "4 to 16 waves");
  static_assert(NT * KPT <= 32 * kBmapWords, "one bitmap bit per block");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  auto sel = gptr(sel_);
  auto cnt = gptr(cnt_);
  const int ibase = wv * 64 * KPT + lane;
  const __amdgpu_buffer_rsrc_t rs = span_rsrc(row, m * 4);
  const __amdgpu_buffer_rsrc_t rt = span_rsrc(trow, m * 4);
  float v[KPT];
  int32_t ph[KPT];
#pragma unroll
  for (int c = 0; c < KPT; ++c)
    v[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (ibase + 64 * c) * 4, 0, 0));
#pragma unroll
  for (int c = 0; c < KPT; ++c) ph[c] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rt, (ibase + 64 * c) * 4, 0, 0);
  const Regions rg = regions_of(ld_uniform_i32(len), initial_len, local_len);
  const int lo = rg.cand_lo, hi = min(rg.cand_hi, m);
  const int n = max(0, hi - lo);
  const int k = min(topk, n);
#ifdef KVS_TIMELINE
  wait_mem();  // the timeline's mark 1: the row has arrived
  if (tl_rec) tl_rec[1] = __builtin_amdgcn_s_memrealtime();
#endif
  if (writer) {
    if (tid == 0) *cnt = k;
    for (int i = k + tid; i < topk; i += NT) sel[i] = -1;
  }
  if (k <= 0) return make_int2(-1, -1);
  const int d = ibase - lo;  // candidate offset of column 0
  uint32_t okb = 0u;
#pragma unroll
  for (int c = 0; c < KPT; ++c) okb |= ((unsigned)(d + 64 * c) < (unsigned)n ? 1u : 0u) << c;
  if (k >= n) {  // every candidate: entry j is block lo + j
#pragma unroll
    for (int c = 0; c < KPT; ++c)
      if ((okb >> c) & 1u) {
        if (writer) sel[d + 64 * c] = ibase + 64 * c;
        if (d + 64 * c == slot) { slot_lds[0] = ibase + 64 * c; slot_lds[1] = ph[c]; }
      }
  } else {
    int off = 0;
    const uint32_t take = topk_reg_take<NT, KPT>(v, okb, k, ibase, S, &off);
    int32_t idv[KPT];
#pragma unroll
    for (int c = 0; c < KPT; ++c) idv[c] = ibase + 64 * c;
    topk_slot_walk<KPT>(take, off, k, idv, ph, slot, slot_lds, writer, sel);
  }
  __syncthreads();
  return slot < k ? make_int2(slot_lds[0], slot_lds[1]) : make_int2(-1, -1);
}

// Selection from chunk summaries.  The candidates of the row are cut into chunks of kChunkBlocks
// blocks, chunk c covering blocks [c * kChunkBlocks, (c + 1) * kChunkBlocks); each chunk's scorer wrote
// its kChunkTop best candidates -- (score, block, physical id), best by (score desc, block asc) --
// sorted by block, padded with (-inf, -1, 0), as uval / uid / uphys[c * kChunkTop + e].  The top k of
// the row are the top k of these entries unless some chunk holds more than kChunkTop of them: that is
// the case exactly when every entry of a chunk with more than kChunkTop candidates is taken, which is
// checked.  The entries are in ascending block order, so the selection comes out in that order.
// summary_take loads the entries (COH: stored by other workgroups of the same kernel, read
// coherently) and finds the taken ones: their bits in *take, the wave's first output slot in *off,
// their block and physical ids in id / ph.  Returns false when a chunk overflows.
template <int NT, int KPT, bool COH>
__device__ __forceinline__ bool summary_take(const float* uval, const int32_t* uid, const int32_t* uphys,
                                             int n_chunks, int cand_lo, int cand_hi, int k, TopkLds& S,
                                             int32_t (&id)[KPT], int32_t (&ph)[KPT], uint32_t* take_out,
                                             int* off_out) {
  static_assert(NT % 256 == 0 && NT <= 1024, "4 to 16 waves");
  static_assert(NT * KPT <= 32 * kBmapWords, "one bitmap bit per entry");
  static_assert(kChunkTop == 8, "a chunk is one byte of a ballot");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int m = n_chunks * kChunkTop;
  const int ibase = wv * 64 * KPT + lane;
  const __amdgpu_buffer_rsrc_t rv = span_rsrc(uval, m * 4);
  const __amdgpu_buffer_rsrc_t ri = span_rsrc(uid, m * 4);
  const __amdgpu_buffer_rsrc_t rp = span_rsrc(uphys, m * 4);
  constexpr int pol = COH ? kSc1 : 0;
  float v[KPT];
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    v[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rv, (ibase + 64 * c) * 4, 0, pol));
    id[c] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(ri, (ibase + 64 * c) * 4, 0, pol);
    ph[c] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rp, (ibase + 64 * c) * 4, 0, pol);
  }
  uint32_t okb = 0u;
#pragma unroll
  for (int c = 0; c < KPT; ++c) okb |= (ibase + 64 * c < m ? 1u : 0u) << c;
  int off = 0;
  const uint32_t take = topk_reg_take<NT, KPT>(v, okb, k, ibase, S, &off);
  // overflow: a chunk (8 consecutive lanes of one column) with every entry taken and more than
  // kChunkTop candidates
  bool ovf = false;
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    const unsigned long long km = __ballot((take >> c) & 1u);
    const int pos = ibase + 64 * c;
    if ((lane & 7) == 0 && pos < m && ((km >> lane) & 0xFFull) == 0xFFull) {
      const int ch = pos / kChunkTop;
      const int n_in = min(cand_hi, (ch + 1) * kChunkBlocks) - max(cand_lo, ch * kChunkBlocks);
      ovf = ovf || n_in > kChunkTop;
    }
  }
  if (tid == 0) S.bcast[0] = 0;
  __syncthreads();
  if (__ballot(ovf) != 0ull && lane == 0) S.bcast[0] = 1;
  __syncthreads();
  *take_out = take;
  *off_out = off;
  return S.bcast[0] == 0;
}

// The selection of the chunk summaries of the same kernel, written in full: sel[0..k) and (with_tiles)
// tiles[0..k).  Returns false, having written nothing, when a chunk overflows (the caller selects from
// the row).
template <int NT, int KPT>
__device__ __forceinline__ bool topk_summary_reg(const float* uval, const int32_t* uid, const int32_t* uphys,
                                                 int n_chunks, int cand_lo, int cand_hi, int k, TopkLds& S,
                                                 int32_t* sel_, int32_t* tiles_, bool with_tiles) {
  int32_t id[KPT], ph[KPT];
  uint32_t take;
  int off;
  if (!summary_take<NT, KPT, true>(uval, uid, uphys, n_chunks, cand_lo, cand_hi, k, S, id, ph, &take, &off))
    return false;
  const int ibase = (threadIdx.x >> 6) * 64 * KPT + (threadIdx.x & 63);
  topk_reg_write<KPT>(take, off, k, ibase, id, true, ph, with_tiles, gptr(sel_), gptr(tiles_));
  return true;
}

// Entry `slot` of the selection from chunk summaries stored by an earlier launch, made by a workgroup
// that attends it (as topk_slot_reg): returns false on a chunk overflow, else true with the entry's
// block and physical id in slot_lds[0..1] once every lane may read them (-1 when slot >= k); with
// `writer` the workgroup also writes sel[0..k).
template <int NT, int KPT>
__device__ __forceinline__ bool topk_summary_slot(const float* uval, const int32_t* uid, const int32_t* uphys,
                                                  int n_chunks, int cand_lo, int cand_hi, int k, int slot,
                                                  TopkLds& S, int* slot_lds, bool writer, int32_t* sel_) {
  int32_t id[KPT], ph[KPT];
  uint32_t take;
  int off;
  if (!summary_take<NT, KPT, false>(uval, uid, uphys, n_chunks, cand_lo, cand_hi, k, S, id, ph, &take, &off))
    return false;
  topk_slot_walk<KPT>(take, off, k, id, ph, slot, slot_lds, writer, gptr(sel_));
  __syncthreads();
  return true;
}

// Selection from a list of preselected blocks: ids[0..m) ascending logical block ids (-1 padded), with
// the score of entry i in vals[i] and its physical id in phys[i], both stored by other workgroups of
// the same kernel (read coherently).  The candidates are the entries with an id in [cand_lo, cand_hi);
// the best k = min(topk, their number) by (score desc, id asc) are written to sel[0..k) (ids,
// ascending) and tiles[0..k) (physical ids), -1 in [k, topk), *cnt = k.
template <int NT, int KPT>
__device__ __forceinline__ void topk_list_reg(const float* vals, const int32_t* phys, const int32_t* ids,
                                              int m, int cand_lo, int cand_hi, int topk, TopkLds& S,
                                              int32_t* sel_, int32_t* cnt_, int32_t* tiles_) {
  static_assert(NT % 256 == 0 && NT <= 1024, "4 to 16 waves");
  static_assert(NT * KPT <= 32 * kBmapWords, "one bitmap bit per entry");
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  auto sel = gptr(sel_);
  auto cnt = gptr(cnt_);
  auto tiles = gptr(tiles_);
  const int ibase = wv * 64 * KPT + lane;
  const __amdgpu_buffer_rsrc_t rv = span_rsrc(vals, m * 4);
  const __amdgpu_buffer_rsrc_t rp = span_rsrc(phys, m * 4);
  const __amdgpu_buffer_rsrc_t ri = span_rsrc(ids, m * 4);
  float v[KPT];
  int32_t id[KPT], ph[KPT];
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    v[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rv, (ibase + 64 * c) * 4, 0, kSc1));
    ph[c] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rp, (ibase + 64 * c) * 4, 0, kSc1);
    id[c] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(ri, (ibase + 64 * c) * 4, 0, 0);
  }
  uint32_t okb = 0u;
  int n_w = 0;  // candidates of this wave
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    const bool ok = ibase + 64 * c < m && id[c] >= cand_lo && id[c] < cand_hi;
    okb |= (ok ? 1u : 0u) << c;
    n_w += __popcll(__ballot(ok));
  }
  if (lane == 0) S.woff[wv] = n_w;
  __syncthreads();
  int n_ok = 0, before = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    n_ok += S.woff[w];
    before += w < wv ? S.woff[w] : 0;
  }
  const int k = min(topk, n_ok);
  uint32_t take = okb;  // every candidate, written in order from the wave's offset
  int off = before;
  if (k < n_ok) take = topk_reg_take<NT, KPT>(v, okb, k, ibase, S, &off);
  if (tid == 0) *cnt = k;
  for (int i = k + tid; i < topk; i += NT) {
    sel[i] = -1;
    tiles[i] = -1;
  }
  if (k > 0) topk_reg_write<KPT>(take, off, k, ibase, id, true, ph, true, sel, tiles);
}

// Entry `slot` of the selection from a preselected list (as topk_list_reg, the list's scores and
// physical ids stored by an earlier launch), made by a workgroup that attends it: returns its block id
// in .x and physical id in .y, or (-1, -1) when slot >= k.  With `writer` the workgroup also writes
// the whole selection: *cnt = k, sel[0..k) ascending, -1 in [k, topk).
template <int NT, int KPT>
__device__ __forceinline__ int2 topk_list_slot(const float* vals, const int32_t* phys, const int32_t* ids,
                                               int m, int cand_lo, int cand_hi, int topk, int slot, TopkLds& S,
                                               int* slot_lds, bool writer, int32_t* sel_, int32_t* cnt_) {
  static_assert(NT % 256 == 0 && NT <= 1024, "4 to 16 waves");
  static_assert(NT * KPT <= 32 * kBmapWords, "one bitmap bit per entry");
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  auto sel = gptr(sel_);
  auto cnt = gptr(cnt_);
  const int ibase = wv * 64 * KPT + lane;
  const __amdgpu_buffer_rsrc_t rv = span_rsrc(vals, m * 4);
  const __amdgpu_buffer_rsrc_t rp = span_rsrc(phys, m * 4);
  const __amdgpu_buffer_rsrc_t ri = span_rsrc(ids, m * 4);
  float v[KPT];
  int32_t id[KPT], ph[KPT];
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    v[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rv, (ibase + 64 * c) * 4, 0, 0));
    ph[c] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rp, (ibase + 64 * c) * 4, 0, 0);
    id[c] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(ri, (ibase + 64 * c) * 4, 0, 0);
  }
  uint32_t okb = 0u;
  int n_w = 0;  // candidates of this wave
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    const bool ok = ibase + 64 * c < m && id[c] >= cand_lo && id[c] < cand_hi;
    okb |= (ok ? 1u : 0u) << c;
    n_w += __popcll(__ballot(ok));
  }
  if (lane == 0) S.woff[wv] = n_w;
  __syncthreads();
  int n_ok = 0, before = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    n_ok += S.woff[w];
    before += w < wv ? S.woff[w] : 0;
  }
  const int k = min(topk, n_ok);
  if (writer) {
    if (tid == 0) *cnt = k;
    for (int i = k + tid; i < topk; i += NT) sel[i] = -1;
  }
  if (k <= 0) return make_int2(-1, -1);
  uint32_t take = okb;  // every candidate, in order from the wave's offset
  int off = before;
  if (k < n_ok) take = topk_reg_take<NT, KPT>(v, okb, k, ibase, S, &off);
  topk_slot_walk<KPT>(take, off, k, id, ph, slot, slot_lds, writer, sel);
  __syncthreads();
  return slot < k ? make_int2(slot_lds[0], slot_lds[1]) : make_int2(-1, -1);
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
  if constexpr (KMAX >= 8) if (max_blocks <= NT * 8) { KVS_TOPK_REG(8); return; }
  if constexpr (KMAX >= 16) if (max_blocks <= NT * 16) { KVS_TOPK_REG(16); return; }
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
