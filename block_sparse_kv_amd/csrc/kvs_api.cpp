// libkvs C ABI: argument validation, workspace sizing and dispatch.  Everything that can be checked
// on the host is checked before the first HIP call, so a rejected call touches neither the device
// nor the stream (and works on a machine without a GPU).
#include <math.h>
#include <stdio.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "kvs.h"
#include "kvs_launch.h"

namespace {

using kvs::Params;

#ifdef KVS_TIMELINE
unsigned long long* g_timeline = nullptr;  // set by kvs_timeline_set
unsigned long long* timeline_records() { return g_timeline; }
#else
unsigned long long* timeline_records() { return nullptr; }
#endif

constexpr size_t kAlign = 256;  // sub-buffers of a workspace start on 256-byte boundaries
constexpr size_t kCtrBytes = kvs::kStepCtrBytes;  // decode-step hand-off counters: batch * G <= 16384

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool pow2_le16(int x) { return x == 1 || x == 2 || x == 4 || x == 8 || x == 16; }

int rep_count_of(const kvs_config* c) {
  switch (c->rep_method) {
    case KVS_REP_QUEST: return 2;
    case KVS_REP_MAX:
    case KVS_REP_MEAN: return 1;
    case KVS_REP_FIX:
      if (c->rep_num < 1 || c->rep_num > c->block_size || c->block_size % c->rep_num) return -1;
      return c->rep_num;
    case KVS_REP_DYNAMIC:
      if (c->rep_num < 1 || c->rep_num > c->block_size) return -1;
      return c->rep_num;
    default: return -1;
  }
}

// Validate a config and fill the kernels' Params.
int make_params(const kvs_config* c, Params* P) {
  if (!c) return KVS_ERR_INVALID_ARG;
  if (c->num_q_heads <= 0 || c->num_kv_heads <= 0 || c->head_dim <= 0 || c->block_size <= 0)
    return KVS_ERR_INVALID_ARG;
  if (c->num_q_heads % c->num_kv_heads) return KVS_ERR_INVALID_ARG;
  if (c->initial_len < 0 || c->local_len < 0 || c->topk < 0) return KVS_ERR_INVALID_ARG;
  if (c->rep_method < KVS_REP_QUEST || c->rep_method > KVS_REP_DYNAMIC) return KVS_ERR_INVALID_ARG;
  if (c->head_select_mode != KVS_HEADS_SEPARATE && c->head_select_mode != KVS_HEADS_SHARED)
    return KVS_ERR_INVALID_ARG;
  if (!(c->softmax_scale >= 0.f) || isinf(c->softmax_scale)) return KVS_ERR_INVALID_ARG;
  if (c->kv_type != KVS_KV_FP16 && c->kv_type != KVS_KV_Q8_0 && c->kv_type != KVS_KV_Q4_0 &&
      c->kv_type != KVS_KV_INT8_PTH && c->kv_type != KVS_KV_INT4_PTH)
    return KVS_ERR_INVALID_ARG;
  const int R = rep_count_of(c);
  if (R < 0) return KVS_ERR_INVALID_ARG;
  if (c->head_dim != kvs::kDim || c->block_size != kvs::kBlock) return KVS_ERR_UNSUPPORTED;
  const int g = c->num_q_heads / c->num_kv_heads;
  if (!pow2_le16(c->num_kv_heads) || !pow2_le16(g)) return KVS_ERR_UNSUPPORTED;
  P->Hq = c->num_q_heads;
  P->Hkv = c->num_kv_heads;
  P->g = g;
  P->G = c->head_select_mode == KVS_HEADS_SEPARATE ? c->num_kv_heads : 1;
  P->initial_len = c->initial_len;
  P->local_len = c->local_len;
  P->topk = c->topk;
  P->method = c->rep_method;
  P->R = R;
  P->mode = c->head_select_mode;
  const float scale = c->softmax_scale > 0.f ? c->softmax_scale : 1.0f / sqrtf((float)c->head_dim);
  P->scale_log2 = scale * 1.4426950408889634f;
  P->kv = c->kv_type;
  P->tl = timeline_records();
  P->tl_kind = 0;
  return KVS_OK;
}

int check_sizes(int32_t batch, int32_t max_blocks) {
  if (batch <= 0 || max_blocks <= 0) return KVS_ERR_INVALID_ARG;
  return KVS_OK;
}

thread_local char g_last_error[512] = "";

int hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return KVS_OK;
  snprintf(g_last_error, sizeof g_last_error, "%s: %s (%s)", where, hipGetErrorName(e),
           hipGetErrorString(e));
  return KVS_ERR_HIP;
}

// Clear a launch error left by earlier, unrelated HIP work so it is not reported as ours.
void clear_stale_error() { (void)hipGetLastError(); }

// Workspace of the attention: the per-tile partials.
struct AttnLayout {
  kvs::AttnPlan plan;
  size_t part_o_off, part_ml_off, total;
};

AttnLayout attn_layout(const Params& P, int batch, int max_blocks) {
  AttnLayout a;
  a.plan = kvs::attn_plan(P, batch, max_blocks);
  size_t off = 0;
  a.part_o_off = off;  off += round_up(a.plan.part_o_bytes);
  a.part_ml_off = off; off += round_up(a.plan.part_ml_bytes);
  a.total = off;
  return a;
}

// Workspace of the decode step: hand-off counters (zero between calls), scores, the selection (when
// the caller does not take it), the selected tiles' physical ids, then the attention partials.
struct StepLayout {
  AttnLayout attn;
  size_t ctr_off, scores_off, sel_off, cnt_off, tiles_off, summ_off, summ_bytes, attn_off, total;
};

StepLayout step_layout(const Params& P, int batch, int max_blocks) {
  StepLayout s;
  const size_t nsel = (size_t)batch * P.G * (P.topk > 0 ? P.topk : 1) * sizeof(int32_t);
  size_t off = 0;
  s.ctr_off = off;    off += kCtrBytes;  // fixed, so every call finds its counters in the zeroed area
  s.scores_off = off; off += round_up((size_t)batch * P.G * max_blocks * sizeof(float));
  s.sel_off = off;    off += round_up(nsel);
  s.cnt_off = off;    off += round_up((size_t)batch * P.G * sizeof(int32_t));
  s.tiles_off = off;  off += round_up(nsel);
  s.summ_bytes = kvs::summaries_bytes(P, batch, max_blocks);  // chunk summaries: scores, ids, physical ids
  s.summ_off = off;   off += 3 * round_up(s.summ_bytes);
  s.attn = attn_layout(P, batch, max_blocks);
  s.attn_off = off;   off += s.attn.total;
  s.total = off;
  return s;
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

kvs::AttnArgs attn_args(const Params& P, const AttnLayout& L, void* ws, const void* q,
                        const void* k_pool, const void* v_pool, const int32_t* table, int max_blocks,
                        const int32_t* seq_lens, const int32_t* sel, const int32_t* sel_count,
                        float* out) {
  kvs::AttnArgs a;
  a.P = P;
  a.q = static_cast<const uint16_t*>(q);
  a.k_pool = static_cast<const uint16_t*>(k_pool);
  a.v_pool = static_cast<const uint16_t*>(v_pool);
  a.table = table;
  a.seq_lens = seq_lens;
  a.sel = sel;
  a.sel_count = sel_count;
  a.part_o = at<float>(ws, L.part_o_off);
  a.part_ml = at<float>(ws, L.part_ml_off);
  a.out = out;
  a.max_blocks = max_blocks;
  a.n_il_max = L.plan.n_il_max;
  a.max_parts = L.plan.max_parts;
  return a;
}

// ---- device contents (KVS_DEBUG=1) -------------------------------------------------------------
// The checks of kvs_validate_contents, on host arrays; each failure names the first bad entry.
int fail_contents(const char* what, long i, long j, long v) {
  snprintf(g_last_error, sizeof g_last_error, "kvs contents: %s at [%ld][%ld] = %ld", what, i, j, v);
  return KVS_ERR_INVALID_ARG;
}

int validate_host(const Params& P, const int32_t* lens, int batch, const int32_t* table, int max_blocks,
                  const int32_t* sel, const int32_t* cnt, const int32_t* presel, int n_presel) {
  for (int i = 0; i < batch; ++i) {
    const int L = lens[i];
    if (L < 1 || (long)L > (long)max_blocks * kvs::kBlock) return fail_contents("seq_len out of [1, max_blocks*128]", i, 0, L);
    const int nb = (L + kvs::kBlock - 1) / kvs::kBlock;
    if (table)
      for (int b = 0; b < nb; ++b)
        if (table[(size_t)i * max_blocks + b] < 0) return fail_contents("block_table entry < 0", i, b, table[(size_t)i * max_blocks + b]);
    const kvs::Regions rg = kvs::regions_of(L, P.initial_len, P.local_len);
    const int n_cand = rg.cand_hi - rg.cand_lo;
    for (int gi = 0; gi < P.G; ++gi) {
      const size_t row = (size_t)i * P.G + gi;
      if (cnt) {
        const int c = cnt[row];
        if (c < 0 || c > P.topk || c > n_cand) return fail_contents("sel_count out of [0, min(topk, candidates)]", (long)row, 0, c);
        if (sel) {
          std::vector<char> seen(max_blocks, 0);
          for (int e = 0; e < c; ++e) {
            const int b = sel[row * P.topk + e];
            if (b < rg.cand_lo || b >= rg.cand_hi) return fail_contents("selected block not a candidate", (long)row, e, b);
            if (seen[b]) return fail_contents("selected block repeated", (long)row, e, b);
            seen[b] = 1;
          }
        }
      }
      if (presel)
        for (int e = 0; e < n_presel; ++e) {
          const int b = presel[row * n_presel + e];
          if (b < -1 || b >= max_blocks) return fail_contents("preselected block out of [-1, max_blocks)", (long)row, e, b);
        }
    }
  }
  return KVS_OK;
}

bool debug_on() {
  const char* e = getenv("KVS_DEBUG");
  return e && e[0] && strcmp(e, "0") != 0;
}

// KVS_DEBUG=1: wait for `stream`, copy the device arrays that steer the kernels to the host and
// validate them before anything is enqueued.  Skipped while the stream is being captured into a graph
// (nothing can be waited for then).  Null arrays are not checked.
int debug_check(const Params& P, hipStream_t s, const int32_t* lens_d, int batch, const int32_t* table_d,
                int max_blocks, const int32_t* sel_d, const int32_t* cnt_d, const int32_t* presel_d,
                int n_presel) {
  if (!debug_on()) return KVS_OK;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return KVS_OK;
  hipError_t e = hipStreamSynchronize(s);
  const size_t rows = (size_t)batch * P.G;
  std::vector<int32_t> lens(batch), table(table_d ? (size_t)batch * max_blocks : 0),
      sel(sel_d ? rows * P.topk : 0), cnt(cnt_d ? rows : 0), presel(presel_d ? rows * n_presel : 0);
  auto copy = [&](std::vector<int32_t>& h, const int32_t* d) {
    if (e == hipSuccess && d && !h.empty())
      e = hipMemcpy(h.data(), d, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost);
  };
  copy(lens, lens_d);
  copy(table, table_d);
  copy(sel, sel_d);
  copy(cnt, cnt_d);
  copy(presel, presel_d);
  if (e != hipSuccess) return hip_status(e, "KVS_DEBUG contents check");
  return validate_host(P, lens.data(), batch, table_d ? table.data() : nullptr, max_blocks,
                       sel_d ? sel.data() : nullptr, cnt_d ? cnt.data() : nullptr,
                       presel_d ? presel.data() : nullptr, n_presel);
}

// Physical block ids of kvs_build_reps / kvs_quantize_kv must not be negative.
int debug_check_ids(hipStream_t s, const int32_t* ids_d, int n) {
  if (!debug_on()) return KVS_OK;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return KVS_OK;
  std::vector<int32_t> ids(n);
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipMemcpy(ids.data(), ids_d, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_status(e, "KVS_DEBUG contents check");
  for (int i = 0; i < n; ++i)
    if (ids[i] < 0) return fail_contents("physical block id < 0", i, 0, ids[i]);
  return KVS_OK;
}

// ---- the allocation-free decode step ----------------------------------------------------------
// A file-scope device array holds the decode-step workspace for callers that cannot allocate.  Each
// GPU holds its own copy until the process ends; host code reaches it only through the address
// hipGetSymbolAddress returns for the current device (the array's name is a host-side stand-in).
constexpr size_t kScratchBytes = KVS_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch sub-buffers are 256-byte aligned");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Zero the hand-off counters (a fill kernel, not a memset node, so a captured first call replays
// correctly).
__global__ void zero_ctr_kernel(unsigned* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// The scratch address on the current device, set up on the first call there: the symbol's address,
// and its counters cleared on `s` (the array starts zeroed; a clear also covers a module loaded into
// a context that reuses memory).
int scratch_on_device(hipStream_t s, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "kvs_decode_step_noalloc/hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return KVS_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol,
                                                 "kvs_decode_step_noalloc/hipGetSymbolAddress");
    hipLaunchKernelGGL(zero_ctr_kernel, dim3(16), dim3(256), 0, s, static_cast<unsigned*>(p),
                       (int)(kCtrBytes / sizeof(unsigned)));
    e = hipGetLastError();
    if (e != hipSuccess) return hip_status(e, "kvs_decode_step_noalloc/clear");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KVS_OK;
}

}  // namespace

extern "C" {

int kvs_validate_contents(const kvs_config* cfg, const int32_t* seq_lens, int32_t batch,
                          const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* sel,
                          const int32_t* sel_count, const int32_t* presel, int32_t n_presel) {
  Params P;
  int st = make_params(cfg, &P);
  if (st != KVS_OK) return st;
  if ((st = check_sizes(batch, max_blocks_per_seq)) != KVS_OK) return st;
  if (!seq_lens || (sel && !sel_count) || (presel && n_presel < 1)) return KVS_ERR_INVALID_ARG;
  return validate_host(P, seq_lens, batch, block_table, max_blocks_per_seq, sel, sel_count, presel, n_presel);
}

const char* kvs_last_error(void) { return g_last_error; }

const char* kvs_status_string(int status) {
  switch (status) {
    case KVS_OK: return "KVS_OK";
    case KVS_ERR_INVALID_ARG: return "KVS_ERR_INVALID_ARG: null pointer, negative size or inconsistent shapes";
    case KVS_ERR_UNSUPPORTED: return "KVS_ERR_UNSUPPORTED: shape outside head_dim=128, block_size=128, Hkv in {1,2,4,8,16}, Hq/Hkv in {1,2,4,8,16}";
    case KVS_ERR_MISALIGNED: return "KVS_ERR_MISALIGNED: q, pools and rep_pool need 16-byte alignment, workspace 256-byte";
    case KVS_ERR_WORKSPACE: return "KVS_ERR_WORKSPACE: workspace null or too small";
    case KVS_ERR_HIP: return "KVS_ERR_HIP: kernel launch failed";
    default: return "unknown kvs status";
  }
}

int kvs_rep_count(const kvs_config* cfg) {
  Params P;
  const int st = make_params(cfg, &P);
  return st == KVS_OK ? P.R : st;
}

size_t kvs_rep_bytes_per_block(const kvs_config* cfg) {
  Params P;
  if (make_params(cfg, &P) != KVS_OK) return 0;
  const size_t elem = P.method == kvs::kMean ? 4 : 2;
  return (size_t)P.Hkv * P.R * kvs::kDim * elem;
}

size_t kvs_kv_bytes_per_block(const kvs_config* cfg) {
  Params P;
  if (make_params(cfg, &P) != KVS_OK) return 0;
  const size_t rec = P.kv == kvs::kKvQ8   ? (size_t)kvs::kQ8Record
                     : P.kv == kvs::kKvQ4 ? (size_t)kvs::kQ4Record
                     : P.kv == kvs::kKvI8 ? (size_t)kvs::kI8Record
                     : P.kv == kvs::kKvI4 ? (size_t)kvs::kI4Record
                                          : (size_t)kvs::kTile * 2;
  return (size_t)P.Hkv * rec;
}

int kvs_quantize_kv(const kvs_config* cfg, const void* src_pool, const int32_t* phys_block_ids,
                    int32_t n_blocks, void* dst_pool, kvs_stream_t stream) {
  Params P;
  int st = make_params(cfg, &P);
  if (st != KVS_OK) return st;
  if (P.kv == kvs::kKvFp16 || n_blocks < 0) return KVS_ERR_INVALID_ARG;
  if (n_blocks == 0) return KVS_OK;
  if (n_blocks > 65535) return KVS_ERR_UNSUPPORTED;  // grid y
  if (!src_pool || !phys_block_ids || !dst_pool) return KVS_ERR_INVALID_ARG;
  if (!aligned(src_pool, 16) || !aligned(dst_pool, 16)) return KVS_ERR_MISALIGNED;
  if ((st = debug_check_ids(static_cast<hipStream_t>(stream), phys_block_ids, n_blocks)) != KVS_OK) return st;
  clear_stale_error();
  return hip_status(kvs::launch_quantize_q8(P, src_pool, phys_block_ids, n_blocks, dst_pool,
                                            static_cast<hipStream_t>(stream)),
                    "kvs_quantize_kv");
}

int kvs_build_reps(const kvs_config* cfg, const void* k_pool, const int32_t* phys_block_ids,
                   int32_t n_blocks, void* rep_pool, kvs_stream_t stream) {
  Params P;
  int st = make_params(cfg, &P);
  if (st != KVS_OK) return st;
  if (n_blocks < 0 || P.method == kvs::kDynamic) return KVS_ERR_INVALID_ARG;
  if (n_blocks == 0) return KVS_OK;
  if (!k_pool || !phys_block_ids || !rep_pool) return KVS_ERR_INVALID_ARG;
  if (!aligned(k_pool, 16) || !aligned(rep_pool, 16)) return KVS_ERR_MISALIGNED;
  if ((st = debug_check_ids(static_cast<hipStream_t>(stream), phys_block_ids, n_blocks)) != KVS_OK) return st;
  clear_stale_error();
  return hip_status(kvs::launch_build_reps(P, k_pool, phys_block_ids, n_blocks, cfg->rep_num,
                                           rep_pool, static_cast<hipStream_t>(stream)),
                    "kvs_build_reps");
}

size_t kvs_importance_workspace_size(const kvs_config* cfg, int32_t batch, int32_t max_blocks_per_seq,
                                     int32_t n_obs) {
  Params P;
  if (make_params(cfg, &P) != KVS_OK || check_sizes(batch, max_blocks_per_seq) != KVS_OK) return 0;
  if (n_obs < 1 || n_obs > 4096) return 0;
  return round_up(kvs::token_importance_ws_bytes(P, batch, max_blocks_per_seq, n_obs));
}

int kvs_token_importance(const kvs_config* cfg, const void* q_obs, int32_t n_obs, const void* k_pool,
                         const int32_t* block_table, int32_t max_blocks_per_seq,
                         const int32_t* seq_lens, int32_t batch, float* importance, void* workspace,
                         size_t workspace_bytes, kvs_stream_t stream) {
  Params P;
  int st = make_params(cfg, &P);
  if (st != KVS_OK) return st;
  if ((st = check_sizes(batch, max_blocks_per_seq)) != KVS_OK) return st;
  if (n_obs < 1) return KVS_ERR_INVALID_ARG;
  if (n_obs > 4096 || batch > 65535 || P.Hkv > 65535) return KVS_ERR_UNSUPPORTED;
  if (!q_obs || !k_pool || !block_table || !seq_lens || !importance) return KVS_ERR_INVALID_ARG;
  if (!aligned(q_obs, 16) || !aligned(k_pool, 16)) return KVS_ERR_MISALIGNED;
  const size_t need = round_up(kvs::token_importance_ws_bytes(P, batch, max_blocks_per_seq, n_obs));
  if (!workspace || workspace_bytes < need) return KVS_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return KVS_ERR_MISALIGNED;
  if ((st = debug_check(P, static_cast<hipStream_t>(stream), seq_lens, batch, block_table, max_blocks_per_seq, nullptr, nullptr, nullptr, 0)) != KVS_OK) return st;
  clear_stale_error();
  return hip_status(kvs::launch_token_importance(P, q_obs, n_obs, k_pool, block_table, max_blocks_per_seq,
                                                 seq_lens, batch, importance, workspace,
                                                 static_cast<hipStream_t>(stream)),
                    "kvs_token_importance");
}

int kvs_build_dynamic_reps(const kvs_config* cfg, const void* k_pool, const float* importance,
                           const int32_t* block_table, int32_t max_blocks_per_seq,
                           const int32_t* seq_lens, int32_t batch, void* rep_pool,
                           kvs_stream_t stream) {
  Params P;
  int st = make_params(cfg, &P);
  if (st != KVS_OK) return st;
  if ((st = check_sizes(batch, max_blocks_per_seq)) != KVS_OK) return st;
  if (P.method != kvs::kDynamic) return KVS_ERR_INVALID_ARG;
  if (batch > 65535) return KVS_ERR_UNSUPPORTED;
  if (!k_pool || !importance || !block_table || !seq_lens || !rep_pool) return KVS_ERR_INVALID_ARG;
  if (!aligned(k_pool, 16) || !aligned(rep_pool, 16)) return KVS_ERR_MISALIGNED;
  if ((st = debug_check(P, static_cast<hipStream_t>(stream), seq_lens, batch, block_table, max_blocks_per_seq, nullptr, nullptr, nullptr, 0)) != KVS_OK) return st;
  clear_stale_error();
  return hip_status(kvs::launch_dynamic_reps(P, k_pool, importance, block_table, max_blocks_per_seq,
                                             seq_lens, batch, rep_pool, static_cast<hipStream_t>(stream)),
                    "kvs_build_dynamic_reps");
}

int kvs_score_blocks(const kvs_config* cfg, const void* q, const void* rep_pool,
                     const int32_t* block_table, int32_t max_blocks_per_seq,
                     const int32_t* seq_lens, int32_t batch, float* scores, kvs_stream_t stream) {
  Params P;
  int st = make_params(cfg, &P);
  if (st != KVS_OK) return st;
  if ((st = check_sizes(batch, max_blocks_per_seq)) != KVS_OK) return st;
  if (!q || !rep_pool || !block_table || !seq_lens || !scores) return KVS_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(rep_pool, 16)) return KVS_ERR_MISALIGNED;
  if ((st = debug_check(P, static_cast<hipStream_t>(stream), seq_lens, batch, block_table, max_blocks_per_seq, nullptr, nullptr, nullptr, 0)) != KVS_OK) return st;
  clear_stale_error();
  return hip_status(kvs::launch_score(P, q, rep_pool, block_table, max_blocks_per_seq, seq_lens,
                                      batch, scores, static_cast<hipStream_t>(stream)),
                    "kvs_score_blocks");
}

int kvs_topk_blocks(const kvs_config* cfg, const float* scores, const int32_t* seq_lens,
                    int32_t batch, int32_t max_blocks_per_seq, int32_t* sel, int32_t* sel_count,
                    kvs_stream_t stream) {
  Params P;
  int st = make_params(cfg, &P);
  if (st != KVS_OK) return st;
  if ((st = check_sizes(batch, max_blocks_per_seq)) != KVS_OK) return st;
  if (!scores || !seq_lens || !sel_count || (!sel && P.topk > 0)) return KVS_ERR_INVALID_ARG;
  if ((st = debug_check(P, static_cast<hipStream_t>(stream), seq_lens, batch, nullptr, max_blocks_per_seq, nullptr, nullptr, nullptr, 0)) != KVS_OK) return st;
  clear_stale_error();
  return hip_status(kvs::launch_topk(P, scores, seq_lens, batch, max_blocks_per_seq, sel,
                                     sel_count, nullptr, nullptr, static_cast<hipStream_t>(stream)),
                    "kvs_topk_blocks");
}

size_t kvs_attn_workspace_size(const kvs_config* cfg, int32_t batch, int32_t max_blocks_per_seq) {
  Params P;
  if (make_params(cfg, &P) != KVS_OK || check_sizes(batch, max_blocks_per_seq) != KVS_OK) return 0;
  return attn_layout(P, batch, max_blocks_per_seq).total;
}

int kvs_sparse_decode_attn(const kvs_config* cfg, const void* q, const void* k_pool,
                           const void* v_pool, const int32_t* block_table,
                           int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                           const int32_t* sel, const int32_t* sel_count, float* out,
                           void* workspace, size_t workspace_bytes, kvs_stream_t stream) {
  Params P;
  int st = make_params(cfg, &P);
  if (st != KVS_OK) return st;
  if ((st = check_sizes(batch, max_blocks_per_seq)) != KVS_OK) return st;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !sel_count || !out ||
      (!sel && P.topk > 0))
    return KVS_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16)) return KVS_ERR_MISALIGNED;
  const AttnLayout A = attn_layout(P, batch, max_blocks_per_seq);
  if (!workspace || workspace_bytes < A.total) return KVS_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return KVS_ERR_MISALIGNED;
  kvs::AttnArgs a = attn_args(P, A, workspace, q, k_pool, v_pool, block_table, max_blocks_per_seq,
                              seq_lens, sel, sel_count, out);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = debug_check(P, s, seq_lens, batch, block_table, max_blocks_per_seq, P.topk > 0 ? sel : nullptr, sel_count, nullptr, 0)) != KVS_OK) return st;
  clear_stale_error();
  hipError_t e = kvs::launch_attn_tiles(a, batch, true, false, s);
  if (e != hipSuccess) return hip_status(e, "kvs_sparse_decode_attn/tiles");
  return hip_status(kvs::launch_merge(a, batch, s), "kvs_sparse_decode_attn/merge");
}

int kvs_gather_read_floor(const void* k_pool, const void* v_pool, int32_t pool_tiles,
                          const int32_t* tile_ids, int32_t n_tiles, int32_t lds_bytes, float* out,
                          kvs_stream_t stream) {
  if (n_tiles < 0 || pool_tiles < 0 || lds_bytes < 0 || lds_bytes > 65536) return KVS_ERR_INVALID_ARG;
  if (n_tiles == 0) return KVS_OK;
  if (!k_pool || !v_pool || !tile_ids || !out) return KVS_ERR_INVALID_ARG;
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16)) return KVS_ERR_MISALIGNED;
  clear_stale_error();
  return hip_status(kvs::launch_gather_read(k_pool, v_pool, pool_tiles, tile_ids, n_tiles, lds_bytes, out,
                                            static_cast<hipStream_t>(stream)),
                    "kvs_gather_read_floor");
}

size_t kvs_decode_step_workspace_size(const kvs_config* cfg, int32_t batch,
                                      int32_t max_blocks_per_seq) {
  Params P;
  if (make_params(cfg, &P) != KVS_OK || check_sizes(batch, max_blocks_per_seq) != KVS_OK) return 0;
  return step_layout(P, batch, max_blocks_per_seq).total;
}

}  // extern "C"

namespace {
// Host checks of kvs_decode_step's arguments other than the workspace.
int decode_step_checks(const kvs_config* cfg, Params* P, const void* q, const void* k_pool,
                       const void* v_pool, const void* rep_pool, const int32_t* block_table,
                       int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch, float* out) {
  int st = make_params(cfg, P);
  if (st != KVS_OK) return st;
  if ((st = check_sizes(batch, max_blocks_per_seq)) != KVS_OK) return st;
  if (!q || !k_pool || !v_pool || !rep_pool || !block_table || !seq_lens || !out)
    return KVS_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(rep_pool, 16))
    return KVS_ERR_MISALIGNED;
  if ((size_t)batch * P->G * sizeof(int) > kCtrBytes) return KVS_ERR_UNSUPPORTED;
  return KVS_OK;
}

// The decode step over a checked workspace of at least step_layout(...).total bytes.
int decode_step_run(const Params& P, const void* q, const void* k_pool, const void* v_pool,
                    const void* rep_pool, const int32_t* block_table, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, int32_t batch, float* out, int32_t* sel_out,
                    int32_t* sel_count_out, void* workspace, hipStream_t s, const char* where) {
  const StepLayout S = step_layout(P, batch, max_blocks_per_seq);
  int32_t* sel = sel_out ? sel_out : at<int32_t>(workspace, S.sel_off);
  int32_t* cnt = sel_count_out ? sel_count_out : at<int32_t>(workspace, S.cnt_off);
  int32_t* tiles = at<int32_t>(workspace, S.tiles_off);
  float* scores = at<float>(workspace, S.scores_off);
  void* aws = static_cast<char*>(workspace) + S.attn_off;
  kvs::AttnArgs a = attn_args(P, S.attn, aws, q, k_pool, v_pool, block_table, max_blocks_per_seq,
                              seq_lens, tiles, cnt, out);
  clear_stale_error();
  return hip_status(kvs::launch_decode_step(a, rep_pool, scores, sel, cnt, tiles,
                                            at<int>(workspace, S.ctr_off), batch, s,
                                            S.summ_bytes ? at<char>(workspace, S.summ_off) : nullptr),
                    where);
}
}  // namespace

extern "C" {

int kvs_decode_step(const kvs_config* cfg, const void* q, const void* k_pool, const void* v_pool,
                    const void* rep_pool, const int32_t* block_table, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, int32_t batch, float* out, int32_t* sel_out,
                    int32_t* sel_count_out, void* workspace, size_t workspace_bytes,
                    kvs_stream_t stream) {
  Params P;
  int st = decode_step_checks(cfg, &P, q, k_pool, v_pool, rep_pool, block_table, max_blocks_per_seq,
                              seq_lens, batch, out);
  if (st != KVS_OK) return st;
  const StepLayout S = step_layout(P, batch, max_blocks_per_seq);
  if (!workspace || workspace_bytes < S.total) return KVS_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return KVS_ERR_MISALIGNED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = debug_check(P, s, seq_lens, batch, block_table, max_blocks_per_seq, nullptr, nullptr, nullptr, 0)) != KVS_OK) return st;
  return decode_step_run(P, q, k_pool, v_pool, rep_pool, block_table, max_blocks_per_seq, seq_lens,
                         batch, out, sel_out, sel_count_out, workspace, s, "kvs_decode_step");
}

int kvs_decode_step_noalloc(const kvs_config* cfg, const void* q, const void* k_pool, const void* v_pool,
                            const void* rep_pool, const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, int32_t batch, float* out, int32_t* sel_out,
                            int32_t* sel_count_out, kvs_stream_t stream) {
  Params P;
  int st = decode_step_checks(cfg, &P, q, k_pool, v_pool, rep_pool, block_table, max_blocks_per_seq,
                              seq_lens, batch, out);
  if (st != KVS_OK) return st;
  const StepLayout S = step_layout(P, batch, max_blocks_per_seq);
  if (S.total > kScratchBytes) {
    snprintf(g_last_error, sizeof g_last_error,
             "kvs_decode_step_noalloc: these sizes need %zu bytes of scratch; the static scratch holds %zu "
             "(use kvs_decode_step with a workspace)", S.total, kScratchBytes);
    return KVS_ERR_WORKSPACE;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = debug_check(P, s, seq_lens, batch, block_table, max_blocks_per_seq, nullptr, nullptr, nullptr, 0)) != KVS_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_on_device(s, &ws)) != KVS_OK) return st;
  return decode_step_run(P, q, k_pool, v_pool, rep_pool, block_table, max_blocks_per_seq, seq_lens,
                         batch, out, sel_out, sel_count_out, ws, s, "kvs_decode_step_noalloc");
}

size_t kvs_preselect_workspace_size(const kvs_config* cfg, int32_t batch, int32_t max_blocks_per_seq) {
  Params P;
  if (make_params(cfg, &P) != KVS_OK || check_sizes(batch, max_blocks_per_seq) != KVS_OK) return 0;
  return round_up((size_t)batch * P.G * max_blocks_per_seq * sizeof(float));
}

int kvs_preselect_blocks(const kvs_config* cfg, const float* importance, const int32_t* seq_lens,
                         int32_t batch, int32_t max_blocks_per_seq, int32_t n_presel,
                         int32_t pool_kernel, int32_t* presel,
                         int32_t* presel_count, void* workspace, size_t workspace_bytes,
                         kvs_stream_t stream) {
  Params P;
  int st = make_params(cfg, &P);
  if (st != KVS_OK) return st;
  if ((st = check_sizes(batch, max_blocks_per_seq)) != KVS_OK) return st;
  if (n_presel < 1) return KVS_ERR_INVALID_ARG;
  if (pool_kernel < 0 || pool_kernel > 127 || (pool_kernel > 0 && pool_kernel % 2 == 0))
    return KVS_ERR_INVALID_ARG;
  if (batch > 65535) return KVS_ERR_UNSUPPORTED;
  if (!importance || !seq_lens || !presel || !presel_count) return KVS_ERR_INVALID_ARG;
  if (!aligned(importance, 16)) return KVS_ERR_MISALIGNED;
  const size_t need = round_up((size_t)batch * P.G * max_blocks_per_seq * sizeof(float));
  if (!workspace || workspace_bytes < need) return KVS_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return KVS_ERR_MISALIGNED;
  float* bs = static_cast<float*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = debug_check(P, s, seq_lens, batch, nullptr, max_blocks_per_seq, nullptr, nullptr, nullptr, 0)) != KVS_OK) return st;
  clear_stale_error();
  hipError_t e = kvs::launch_block_scores(P, importance, seq_lens, batch, max_blocks_per_seq, pool_kernel,
                                         bs, s);
  if (e != hipSuccess) return hip_status(e, "kvs_preselect_blocks/scores");
  Params Q = P;
  Q.topk = n_presel;
  return hip_status(kvs::launch_topk(Q, bs, seq_lens, batch, max_blocks_per_seq, presel, presel_count,
                                     nullptr, nullptr, s),
                    "kvs_preselect_blocks/top-k");
}

namespace {
// Workspace of the confined decode step: scores, the compacted rows (scores, block ids, lengths),
// their top-k picks, the selection and counts when the caller does not take them, then the partials.
// Workspace of the confined step: hand-off counters (zero between calls) at the start, as in the
// decode step's, then the scores (every candidate, or the sets' entries), the compacted rows, the
// sets' physical ids, the selection and its tiles, and the attention partials.
struct PreselLayout {
  AttnLayout attn;
  size_t ctr_off, scores_off, cs_off, cid_off, cph_off, clen_off, csel_off, sel_off, cnt_off, tiles_off,
      attn_off, total;
};

PreselLayout presel_layout(const Params& P, int batch, int max_blocks, int n_presel) {
  PreselLayout L;
  const size_t rows = (size_t)batch * P.G, k = P.topk > 0 ? P.topk : 1;
  size_t off = 0;
  L.ctr_off = off;    off += kCtrBytes;
  L.scores_off = off; off += round_up(rows * max_blocks * sizeof(float));
  L.cs_off = off;     off += round_up(rows * n_presel * sizeof(float));
  L.cid_off = off;    off += round_up(rows * n_presel * sizeof(int32_t));
  L.cph_off = off;    off += round_up(rows * n_presel * sizeof(int32_t));
  L.clen_off = off;   off += round_up(rows * sizeof(int32_t));
  L.csel_off = off;   off += round_up(rows * k * sizeof(int32_t));
  L.sel_off = off;    off += round_up(rows * k * sizeof(int32_t));
  L.cnt_off = off;    off += round_up(rows * sizeof(int32_t));
  L.tiles_off = off;  off += round_up(rows * k * sizeof(int32_t));
  L.attn = attn_layout(P, batch, max_blocks);
  L.attn_off = off;   off += L.attn.total;
  L.total = off;
  return L;
}
}  // namespace

size_t kvs_decode_step_preselected_workspace_size(const kvs_config* cfg, int32_t batch,
                                                  int32_t max_blocks_per_seq, int32_t n_presel) {
  Params P;
  if (make_params(cfg, &P) != KVS_OK || check_sizes(batch, max_blocks_per_seq) != KVS_OK || n_presel < 1)
    return 0;
  return presel_layout(P, batch, max_blocks_per_seq, n_presel).total;
}

int kvs_decode_step_preselected(const kvs_config* cfg, const void* q, const void* k_pool,
                                const void* v_pool, const void* rep_pool, const int32_t* block_table,
                                int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                                const int32_t* presel, int32_t n_presel, float* out, int32_t* sel_out,
                                int32_t* sel_count_out, void* workspace, size_t workspace_bytes,
                                kvs_stream_t stream) {
  Params P;
  int st = make_params(cfg, &P);
  if (st != KVS_OK) return st;
  if ((st = check_sizes(batch, max_blocks_per_seq)) != KVS_OK) return st;
  if (n_presel < 1) return KVS_ERR_INVALID_ARG;
  if ((size_t)batch * P.G > 65535) return KVS_ERR_UNSUPPORTED;
  if (!q || !k_pool || !v_pool || !rep_pool || !block_table || !seq_lens || !presel || !out)
    return KVS_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(rep_pool, 16))
    return KVS_ERR_MISALIGNED;
  const PreselLayout S = presel_layout(P, batch, max_blocks_per_seq, n_presel);
  if (!workspace || workspace_bytes < S.total) return KVS_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return KVS_ERR_MISALIGNED;
  const int rows = batch * P.G, k = P.topk;
  float* scores = at<float>(workspace, S.scores_off);
  float* cs = at<float>(workspace, S.cs_off);
  int32_t* cid = at<int32_t>(workspace, S.cid_off);
  int32_t* clen = at<int32_t>(workspace, S.clen_off);
  int32_t* csel = at<int32_t>(workspace, S.csel_off);
  int32_t* sel = sel_out ? sel_out : at<int32_t>(workspace, S.sel_off);
  int32_t* cnt = sel_count_out ? sel_count_out : at<int32_t>(workspace, S.cnt_off);
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* aws = static_cast<char*>(workspace) + S.attn_off;
  if ((st = debug_check(P, s, seq_lens, batch, block_table, max_blocks_per_seq, nullptr, nullptr, presel, n_presel)) != KVS_OK) return st;
  if (n_presel <= kvs::presel_step_max() && P.topk > 0 && (size_t)rows * sizeof(int) <= kCtrBytes) {
    // the sets scored, the selections made from them, and every attended tile, in two launches
    int32_t* tiles = at<int32_t>(workspace, S.tiles_off);
    kvs::AttnArgs a = attn_args(P, S.attn, aws, q, k_pool, v_pool, block_table, max_blocks_per_seq,
                                seq_lens, tiles, cnt, out);
    clear_stale_error();
    hipError_t e = kvs::launch_presel_step(a, rep_pool, presel, n_presel, cs, at<int32_t>(workspace, S.cph_off),
                                           sel, cnt, tiles, at<int>(workspace, S.ctr_off), batch, s);
    if (e == hipSuccess) e = kvs::launch_merge(a, batch, s);
    return hip_status(e, "kvs_decode_step_preselected");
  }
  kvs::AttnArgs a = attn_args(P, S.attn, aws, q, k_pool, v_pool, block_table, max_blocks_per_seq,
                              seq_lens, sel, cnt, out);
  clear_stale_error();
  bool il_done = false;  // Initial/Local tiles streamed with the scoring (rows of up to 2048 blocks)
  hipError_t e = kvs::launch_score_il(a, rep_pool, scores, batch, s, &il_done);
  if (n_presel <= 256) {  // the set ranked in one launch
    if (e == hipSuccess)
      e = kvs::launch_presel_select(P, scores, max_blocks_per_seq, seq_lens, presel, n_presel, batch, sel, cnt, s);
  } else {  // compacted rows, each a sequence of its own (n_eff blocks, all candidates), and the top-k
    if (e == hipSuccess)
      e = kvs::launch_compact(P, scores, max_blocks_per_seq, seq_lens, presel, n_presel, batch, cs, cid, clen, s);
    Params C = P;
    C.G = 1;
    C.mode = kvs::kShared;
    C.initial_len = 0;
    C.local_len = 0;
    if (e == hipSuccess) e = kvs::launch_topk(C, cs, clen, rows, n_presel, csel, cnt, nullptr, nullptr, s);
    if (e == hipSuccess) e = kvs::launch_map_back(csel, k, cid, n_presel, rows, sel, s);
  }
  if (e != hipSuccess) return hip_status(e, "kvs_decode_step_preselected/selection");
  e = kvs::launch_attn_tiles(a, batch, !il_done, false, s);
  if (e != hipSuccess) return hip_status(e, "kvs_decode_step_preselected/tiles");
  return hip_status(kvs::launch_merge(a, batch, s), "kvs_decode_step_preselected/merge");
}

#ifdef KVS_TIMELINE
// Timeline build only: the record array (device, kTlKinds * kTlMaxWg * kTlSlots 64-bit words, zeroed
// by the caller) that calls configured from now on write into; null stops recording.
void kvs_timeline_set(void* records) { g_timeline = static_cast<unsigned long long*>(records); }
#endif

}  // extern "C"
