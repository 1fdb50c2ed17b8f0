// kvs_decode_step: one persistent kernel for a whole decode step of one layer
// (KTransformers long-context sparse attention, lmnt.cn, §4.6: retrieval of the relevant blocks,
// then attention over the retrieved cache).
//
// Workgroups claim work items from one ticket counter, in an order where every item only waits for
// items with lower tickets, so progress never depends on which workgroups are resident:
//   1. score items   (sequence, chunk of blocks): block scores of the candidates in the chunk;
//   2. top-k items   (sequence, group): wait for the sequence's score items, select, write the
//                    selection and the physical ids of the selected tiles;
//   3. Initial/Local attention items (sequence, KV head, part): need no selection, so they run while
//                    the top-k items are still working;
//   4. selected attention items (sequence, KV head, part): wait for their group's top-k item.
// Every attention item adds one partial per query head to the workspace and arrives at a counter of
// its (sequence, KV head); the last to arrive merges that head's partials into `out`.
// Data that crosses workgroups (scores, selection, tile ids, partials) is written and read with
// coherent device-scope accesses (st_coh / ld_coh), so a dependency is just: the producer waits for its
// stores to complete, then bumps a device-scope counter; the consumer polls the counter.  No L2
// write-back or invalidate is issued -- on MI355X those act on a whole XCD's L2 and cost tens of
// microseconds each.  Waits are bounded: past the limit the kernel sets an error word and goes on, so
// it always terminates.  The last workgroup to exit zeroes the counters for the next call.
#include "attn_core.h"
#include "kvs_device.h"
#include "kvs_launch.h"
#include "score_core.h"
#include "topk_core.h"

namespace kvs {

constexpr int kStepTopkLdsKeys = 8192;  // candidates staged in LDS by a top-k item
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int kStepSmem = cmax(cmax(kAttnLdsBytes, kStepTopkLdsKeys * 4 + (int)sizeof(TopkLds)),
                               kMergeLdsFloats * 4);
constexpr int kSpinLimit = 1 << 21;  // polls (each a device-scope load plus a short sleep)

__device__ inline int load_count(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until *ctr >= target (thread 0 polls); the data it guards is then read with ld_coh.
__device__ inline void wait_geq(const int* ctr, int target, int* err) {
  if (threadIdx.x == 0) {
    int it = 0;
    while (load_count(ctr) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (++it > kSpinLimit) {
        atomicOr(err, 1);
        break;
      }
    }
  }
  __syncthreads();
}

// After this workgroup's st_coh stores have completed, add 1 to *ctr; returns the count before the
// add (to all lanes).
__device__ inline int release_add(int* ctr, int* s_val) {
  wait_mem();
  __syncthreads();
  if (threadIdx.x == 0)
    *s_val = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return *s_val;
}

template <int G, int METHOD, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void decode_step_kernel(StepArgs A) {
  const Params& P = A.P;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStepSmem];
  __shared__ int s_val;
  const int tid = threadIdx.x;
  int* ctrl = A.ctrl;
  int* score_done = ctrl + kCtrlHead;
  int* topk_done = score_done + A.batch;
  int* attn_done = topk_done + A.batch * P.G;

  for (;;) {
    if (tid == 0) s_val = __hip_atomic_fetch_add(&ctrl[0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int t = s_val;
    __syncthreads();
    if (t >= A.total) break;

    if (t < A.off_topk) {  // ---------------- score item
      const int seq = t / A.n_score_per_seq;
      const int b0 = (t % A.n_score_per_seq) * A.sb;
      const int L = A.seq_lens[seq];
      const Regions rg = regions_of(L, P.initial_len, P.local_len);
      const int lo = max(b0, rg.cand_lo), hi = min(b0 + A.sb, rg.cand_hi);
      if (lo < hi) {
        float* srow = A.scores + (size_t)seq * P.G * A.max_blocks;
        score_blocks_range<G, METHOD, MODE, true>(P, A.q + (size_t)seq * P.Hq * kDim, A.rep_pool,
                                            A.table + (size_t)seq * A.max_blocks, A.max_blocks, L,
                                            lo, hi - lo, srow, reinterpret_cast<float*>(smem));
      }
      release_add(&score_done[seq], &s_val);
    } else if (t < A.off_il) {  // ---------------- top-k item
      const int idx = t - A.off_topk;
      const int seq = idx / P.G, grp = idx % P.G;
      wait_geq(&score_done[seq], A.n_score_per_seq, &ctrl[2]);
      const int L = A.seq_lens[seq];
      const Regions rg = regions_of(L, P.initial_len, P.local_len);
      const int n = rg.cand_hi - rg.cand_lo;
      const int k = min(P.topk, n);
      const size_t row = (size_t)seq * P.G + grp;
      int32_t* sel = A.sel + row * P.topk;
      for (int i = k + tid; i < P.topk; i += 256) st_coh(sel + i, -1);
      if (tid == 0) st_coh(A.sel_count + row, k);
      TopkLds& S = *reinterpret_cast<TopkLds*>(smem + kStepTopkLdsKeys * 4);
      const float* srow = A.scores + row * A.max_blocks + rg.cand_lo;
      const int32_t* trow = A.table + (size_t)seq * A.max_blocks;
      topk_run<256, 32, true>(srow, n, k, rg.cand_lo, reinterpret_cast<uint32_t*>(smem), kStepTopkLdsKeys, S,
                          sel, trow, A.tiles_sel + row * P.topk);
      release_add(&topk_done[row], &s_val);
    } else {  // ---------------- attention items
      const bool il = t < A.off_sel;
      const int idx = il ? t - A.off_il : t - A.off_sel;
      const int per_seq = P.Hkv * (il ? A.n_il_parts : A.n_sel_parts);
      const int seq = idx / per_seq;
      const int h = (idx % per_seq) / (il ? A.n_il_parts : A.n_sel_parts);
      const int p = idx % (il ? A.n_il_parts : A.n_sel_parts);
      const int L = A.seq_lens[seq];
      const Regions rg = regions_of(L, P.initial_len, P.local_len);
      const int32_t* trow = A.table + (size_t)seq * A.max_blocks;
      const size_t head0 = (size_t)seq * P.Hq + (size_t)h * G;
      float* po = A.part_o + head0 * A.n_parts * kDim;
      float* pml = A.part_ml + head0 * A.n_parts * 2;
      const uint16_t* qh = A.q + head0 * kDim;
      if (il) {
        const TileList tl = tiles_of(L, P, 0);  // Initial then Local tiles
        const int nil = tl.nI + tl.nLoc;
        const int t0 = p * A.tps_il;
        const int n = max(0, min(A.tps_il, nil - t0));
        attn_partial<G, true>(P, qh, A.k_pool, A.v_pool, h, n,
                        [&](int i) -> int2 {
                          const int x = t0 + i;
                          const int lb = x < tl.nI ? x : tl.loc_b0 + (x - tl.nI);
                          return make_int2(trow[lb], min(kBlock, L - lb * kBlock));
                        },
                        po, pml, A.n_parts, p, smem);
      } else {
        const int grp = MODE == kSeparate ? h : 0;
        const size_t row = (size_t)seq * P.G + grp;
        const int k = min(P.topk, rg.cand_hi - rg.cand_lo);
        const int t0 = p * A.tps_sel;
        const int n = max(0, min(A.tps_sel, k - t0));
        if (n > 0) wait_geq(&topk_done[row], 1, &ctrl[2]);
        const int32_t* tiles = A.tiles_sel + row * P.topk + t0;
        attn_partial<G, true>(P, qh, A.k_pool, A.v_pool, h, n,
                        [&](int i) -> int2 { return make_int2(ld_coh(tiles + i), kBlock); },
                        po, pml, A.n_parts, A.n_il_parts + p, smem);
      }
      const int before = release_add(&attn_done[(size_t)seq * P.Hkv + h], &s_val);
      if (before == A.n_parts - 1)  // last partial of this (sequence, KV head): merge
        merge_heads<G, true>(po, pml, A.n_parts, A.n_parts, A.out + head0 * kDim,
                             reinterpret_cast<float*>(smem));
    }
  }

  // exit: the last workgroup out resets the counters for the next call
  if (tid == 0) s_val = __hip_atomic_fetch_add(&ctrl[1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (s_val == (int)gridDim.x - 1) {
    const int n_ctr = A.batch + A.batch * P.G + A.batch * P.Hkv;
    for (int i = tid; i < n_ctr; i += 256) st_coh(score_done + i, 0);
    if (tid == 0) { st_coh(ctrl + 0, 0); st_coh(ctrl + 1, 0); }
  }
}

StepPlan step_plan(const Params& P, int batch, int max_blocks, int resident_wgs) {
  StepPlan s;
  const int bpp = 16 / P.Hkv;
  const size_t rep_block = (size_t)P.Hkv * P.R * kDim * (P.method == kMean ? 4 : 2);
  int sb = (int)(65536 / rep_block);  // about 64 KiB of reps per item, loaded in one batch
  sb = max(bpp, min(bpp * kScorePasses, sb)) / bpp * bpp;
  s.sb = sb;
  s.n_score_per_seq = (max_blocks + sb - 1) / sb;
  const int nI = (P.initial_len + kBlock - 1) / kBlock;
  const int nLoc = (P.local_len + 2 * kBlock - 2) / kBlock;
  const int il_max = max(1, min(max_blocks, nI + nLoc));
  const int sel_max = min(P.topk, max_blocks);
  const long tiles = (long)batch * P.Hkv * (il_max + sel_max);
  long tps = (tiles + resident_wgs - 1) / max(1, resident_wgs);
  tps = max(tps, (long)((il_max + sel_max + kMaxParts - 1) / kMaxParts));  // merge bound
  tps = max(1L, min((long)kMaxItemTiles, tps));
  s.tps_il = s.tps_sel = (int)tps;
  s.n_il_parts = (il_max + s.tps_il - 1) / s.tps_il;
  s.n_sel_parts = (sel_max + s.tps_sel - 1) / s.tps_sel;
  s.n_parts = s.n_il_parts + s.n_sel_parts;
  s.off_topk = batch * s.n_score_per_seq;
  s.off_il = s.off_topk + batch * P.G;
  s.off_sel = s.off_il + batch * P.Hkv * s.n_il_parts;
  s.total = s.off_sel + batch * P.Hkv * s.n_sel_parts;
  s.ctrl_ints = kCtrlHead + batch + batch * P.G + batch * P.Hkv;
  s.part_o_bytes = (size_t)batch * P.Hq * s.n_parts * kDim * sizeof(float);
  s.part_ml_bytes = (size_t)batch * P.Hq * s.n_parts * 2 * sizeof(float);
  s.tiles_bytes = (size_t)batch * P.G * max(1, P.topk) * sizeof(int32_t);
  return s;
}

template <int G, int METHOD>
static void* step_kernel_ptr(int mode) {
  return mode == kSeparate ? reinterpret_cast<void*>(&decode_step_kernel<G, METHOD, kSeparate>)
                           : reinterpret_cast<void*>(&decode_step_kernel<G, METHOD, kShared>);
}

template <int G>
static void* step_kernel_g(const Params& P) {
  switch (P.method) {
    case kQuest: return step_kernel_ptr<G, kQuest>(P.mode);
    case kMax: return step_kernel_ptr<G, kMax>(P.mode);
    case kMean: return step_kernel_ptr<G, kMean>(P.mode);
    default: return step_kernel_ptr<G, kFix>(P.mode);
  }
}

static void* step_kernel(const Params& P) {
  switch (P.g) {
    case 1: return step_kernel_g<1>(P);
    case 2: return step_kernel_g<2>(P);
    case 4: return step_kernel_g<4>(P);
    case 8: return step_kernel_g<8>(P);
    default: return step_kernel_g<16>(P);
  }
}

hipError_t step_resident_wgs(const Params& P, int* out) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, step_kernel(P), 256, 0);
  *out = max(1, cus * max(1, per_cu));
  return e;
}

hipError_t launch_step(const StepArgs& A, int grid, hipStream_t s) {
  void* fn = step_kernel(A.P);
  void* args[] = {const_cast<StepArgs*>(&A)};
  return hipLaunchKernel(fn, dim3(grid), dim3(256), args, 0, s);
}

__global__ void zero_words_kernel(int* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 4;
  const int grid = (int)min((size_t)1024, (n + 255) / 256);
  if (grid > 0) hipLaunchKernelGGL(zero_words_kernel, dim3(grid), dim3(256), 0, s, static_cast<int*>(p), n);
  return hipGetLastError();
}

}  // namespace kvs
