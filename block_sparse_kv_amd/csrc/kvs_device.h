// Device-side helpers shared by the libkvs kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvs {

constexpr int kBlock = 128;  // tokens per KV block
constexpr int kDim = 128;    // head_dim
constexpr int kTile = kBlock * kDim;  // fp16 elements in one (block, KV head) tile
// Q8_0 record of one (block, KV head): int8 codes [128 tokens][128], then fp16 scales [128][4]
// (scale [t][c / 32] of channel c of token t).
constexpr int kQ8Group = 32;
constexpr int kQ8Codes = kBlock * kDim;                                // bytes of codes
constexpr int kQ8Record = kQ8Codes + kBlock * (kDim / kQ8Group) * 2;  // 17408 bytes
// Q4_0 record: codes [128 tokens][64 bytes] -- word k of a token row holds channels 8k .. 8k+7,
// channel 8k + 2i in bits 4i..4i+3 and channel 8k + 2i + 1 in bits 16+4i..19+4i -- then fp16 scales
// [128][4] as for Q8_0.
constexpr int kQ4Codes = kBlock * kDim / 2;                            // bytes of codes
constexpr int kQ4Record = kQ4Codes + kBlock * (kDim / kQ8Group) * 2;  // 9216 bytes
// INT8 with one fp32 scale per token row: codes as Q8_0's, then 128 fp32 scales
constexpr int kI8Record = kQ8Codes + kBlock * 4;                       // 16896 bytes
// INT4 with one fp32 scale and one zero point per token row: codes as Q4_0's, then 128 fp32 scales,
// then 128 zero-point bytes
constexpr int kI4Scales = kQ4Codes;                                    // offset of the scales
constexpr int kI4Zeros = kQ4Codes + kBlock * 4;                        // offset of the zero points
constexpr int kI4Record = kI4Zeros + kBlock;                           // 8832 bytes

// Long-row selection from chunk summaries: a chunk is kChunkBlocks consecutive blocks of a score row,
// summarised by its kChunkTop best candidates.
constexpr int kChunkBlocks = 64;
constexpr int kChunkTop = 8;

enum Method { kQuest = 0, kMax = 1, kMean = 2, kFix = 3, kDynamic = 4 };  // Dynamic: scored like Fix
enum Mode { kSeparate = 0, kShared = 1 };
enum KvType { kKvFp16 = 0, kKvQ8 = 1, kKvQ4 = 2, kKvI8 = 3, kKvI4 = 4 };

// Launch-time constants of one call (passed by value to every kernel).
struct Params {
  int Hq, Hkv, g;       // query heads, KV heads, query heads per KV head
  int G;                // selection groups: Hkv (SEPARATE) or 1 (SHARED)
  int initial_len, local_len, topk;
  int method, R, mode;  // rep method, reps per (block, head), head_select_mode
  int kv;               // KvType of the K/V pools
  float scale_log2;     // softmax scale * log2(e): logits live in the exp2 domain
  unsigned long long* tl;  // timeline records (timeline build only; null otherwise)
  int tl_kind;             // TlKind of the tiles of this launch (timeline build only)
};

// Initial / Context / Local split of a sequence of L tokens, rounded outward to whole blocks:
// Initial = [0, init_end), candidates = blocks [cand_lo, cand_hi), Local = [local_start, L).
struct Regions {
  int init_end, local_start, cand_lo, cand_hi;
};

__host__ __device__ inline int floor_div(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

__host__ __device__ inline Regions regions_of(int L, int initial_len, int local_len) {
  Regions r;
  const int ib = ((initial_len + kBlock - 1) / kBlock) * kBlock;
  if (L <= ib) {
    r.init_end = L; r.local_start = L; r.cand_lo = 0; r.cand_hi = 0;
    return r;
  }
  const int lloc = max(ib, floor_div(L - local_len, kBlock) * kBlock);
  r.init_end = ib; r.local_start = lloc; r.cand_lo = ib / kBlock; r.cand_hi = lloc / kBlock;
  return r;
}

// Attended tiles of one selection group: nI Initial tiles, then k selected, then nLoc Local tiles.
struct TileList {
  int nI, k, nLoc, loc_b0, L;
  __device__ int count() const { return nI + k + nLoc; }
};

__device__ inline TileList tiles_of(int L, const Params& P, int k_sel) {
  const Regions rg = regions_of(L, P.initial_len, P.local_len);
  TileList t;
  t.L = L;
  if (L <= rg.init_end) {  // everything is Initial
    t.nI = (L + kBlock - 1) / kBlock; t.k = 0; t.nLoc = 0; t.loc_b0 = 0;
  } else {
    t.nI = rg.init_end / kBlock;
    t.k = max(0, min(k_sel, P.topk));  // a selection never names more than topk blocks
    t.loc_b0 = rg.local_start / kBlock;
    t.nLoc = (L - rg.local_start + kBlock - 1) / kBlock;
  }
  return t;
}

// Logical block and token count of the t-th Initial/Local tile (t < nI + nLoc).
__device__ inline int2 il_tile(const TileList& tl, int t) {
  const int lb = t < tl.nI ? t : tl.loc_b0 + (t - tl.nI);
  return make_int2(lb, min(kBlock, tl.L - lb * kBlock));
}

// Arguments of the attention kernels.  Partials: per (sequence, query head) up to max_parts of them;
// the Initial/Local tiles of a sequence are parts [0, n_il), its selected tiles parts [n_il, n_il + k).
struct AttnArgs {
  Params P;
  const uint16_t* q;         // [batch][Hq][128]
  const uint16_t* k_pool;    // [n_phys][Hkv][128][128]
  const uint16_t* v_pool;
  const int32_t* table;      // [batch][max_blocks]
  const int32_t* seq_lens;   // [batch]
  const int32_t* sel;        // [batch][G][topk]: logical ids, or physical ids (sel_phys)
  const int32_t* sel_count;  // [batch][G]
  float* part_o;             // [batch][Hq][max_parts][128]
  float* part_ml;            // [batch][Hq][max_parts][2]
  float* out;                // [batch][Hq][128]
  int max_blocks, n_il_max, max_parts;
};

// ---- wave64 cross-lane helpers (DPP within 16-lane rows) -----------------------------------------
template <int CTRL>
__device__ inline float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row receives the total.
__device__ inline float row_sum16(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f<0x141>(x);  // row_half_mirror: other quad of the half-row
  x += dpp_f<0x140>(x);  // row_mirror: other half of the row
  return x;
}

__device__ inline float shfl_xor_f(float x, int m) { return __shfl_xor(x, m, 64); }

template <int CTRL>
__device__ inline uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

// Minimum / maximum over the 64 lanes of a wave, the same in every lane: DPP within each 16-lane row,
// then the four row results through readlane (no LDS round trips).
__device__ inline uint32_t wave_min_u32(uint32_t x) {
  x = min(x, dpp_u<0xB1>(x));
  x = min(x, dpp_u<0x4E>(x));
  x = min(x, dpp_u<0x141>(x));
  x = min(x, dpp_u<0x140>(x));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)x, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)x, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  return min(min(a, b), min(c, d));
}
__device__ inline uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_u<0xB1>(x));
  x = max(x, dpp_u<0x4E>(x));
  x = max(x, dpp_u<0x141>(x));
  x = max(x, dpp_u<0x140>(x));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)x, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)x, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  return max(max(a, b), max(c, d));
}

// Float minimum / maximum over the 64 lanes of a wave (NaN lanes are ignored), the same in every lane.
__device__ inline float rl_f(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
__device__ inline float wave_min_f32(float x) {
  x = fminf(x, dpp_f<0xB1>(x));
  x = fminf(x, dpp_f<0x4E>(x));
  x = fminf(x, dpp_f<0x141>(x));
  x = fminf(x, dpp_f<0x140>(x));
  return fminf(fminf(rl_f(x, 0), rl_f(x, 16)), fminf(rl_f(x, 32), rl_f(x, 48)));
}
__device__ inline float wave_max_f32(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));
  x = fmaxf(x, dpp_f<0x4E>(x));
  x = fmaxf(x, dpp_f<0x141>(x));
  x = fmaxf(x, dpp_f<0x140>(x));
  return fmaxf(fmaxf(rl_f(x, 0), rl_f(x, 16)), fmaxf(rl_f(x, 32), rl_f(x, 48)));
}

__device__ inline float wave_sum_f32(float x) {
  x = row_sum16(x);
  return (rl_f(x, 0) + rl_f(x, 16)) + (rl_f(x, 32) + rl_f(x, 48));
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4, 8 inside each 16-lane row,
// then the row totals through the row broadcasts of lanes 15 (into rows 1 and 3) and 31 (into rows
// 2 and 3).
__device__ inline int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// ---- address spaces --------------------------------------------------------------------------------
// A value every lane reads at a uniform address: loaded through the scalar cache.  Only for data no
// workgroup of the running kernel writes.
__device__ inline int ld_uniform_i32(const int32_t* p) {
  typedef __attribute__((address_space(4))) const int32_t cint;
  return *(const cint*)p;
}
// The same pointer, marked global (vector memory instructions rather than flat ones).
template <typename T>
__device__ inline __attribute__((address_space(1))) T* gptr(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}
// Buffer resource over `bytes` bytes from base: loads past the end return 0 (bytes = 0: every load).
__device__ inline __amdgpu_buffer_rsrc_t span_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// ---- fp16 <-> fp32 ----------------------------------------------------------------------------------
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ inline void unpack8(const uint4& v, float (&f)[8]) {
  const half8_t h = __builtin_bit_cast(half8_t, v);
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (float)h[e];
}

__device__ inline uint16_t f2h_bits(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }

// 16-byte streaming load (non-temporal hint: K/V tiles are read once per step).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ inline uint4 ld_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- hand-off between workgroups of one kernel ----------------------------------------------------
// The per-XCD L2 caches are not coherent with each other.  Data one workgroup hands to another of the
// same kernel is written with agent-scope relaxed atomic stores (st_coh: global stores with sc1, which
// write through to the coherence point), the writer waits for their completion (wait_mem: vmcnt 0)
// before its relaxed agent-scope fetch_add on the group's counter, and the workgroup that brings the
// counter to its total reads the data, after a workgroup barrier, with sc1 loads (what agent-scope
// relaxed atomic loads compile to), so it sees the data whichever XCD it runs on.  The ordering rests
// on the ISA: a store counted in vmcnt is complete at the coherence point once vmcnt reads 0, and
// every datum goes through an sc1 access on both sides, so no L2 holds a stale or dirty copy of it.
// A release/acquire pair on the counter would instead write back and invalidate the whole L2 of the
// XCD at every hand-off, which costs several microseconds per decode step.  wait_mem also keeps the
// compiler from moving memory accesses across it (signal fences on both sides).
template <typename T>
__device__ inline void st_coh(T* p, T v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
constexpr int kSc1 = 16;  // cache-policy operand of the raw buffer loads: sc1
__device__ inline __amdgpu_buffer_rsrc_t coh_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}
__device__ inline float ld_coh_f1(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, kSc1));
}
// The per-token-head caches' values are fp32 products that are not exact: keep_fp32 makes one an fp32
// value in a register, so that a later conversion to fp16 rounds it a second time, as the cached value
// is defined, instead of the compiler fusing the product and the conversion into one mixed-precision
// instruction that rounds the exact product once.
__device__ inline void keep_fp32(float& v) { __asm__ volatile("" : "+v"(v)); }

// Wait until this wave's memory operations have completed (vmcnt 0; 0x0F70 leaves expcnt and lgkmcnt
// at their maxima, so only vmcnt is waited on).
__device__ inline void wait_mem() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// exp2(a - b) that is 0 when a is -inf (an empty stream), never NaN.
__device__ inline float exp2_diff(float a, float b) { return a == -INFINITY ? 0.f : fast_exp2(a - b); }

}  // namespace kvs

#include "timeline.h"
