/*
 * kvs.h -- block-sparse long-context decode attention over a paged fp16 KV cache, for AMD MI355X
 * (gfx950).  C ABI of libkvs.so.
 *
 * The method is the one the KTransformers long-context sparse-attention article describes
 * ("KTransformers 长上下文稀疏注意力实战", lmnt.cn; cited below as [KT-LC §n]):
 *   1. per-block representative keys ("reps") built once per filled block           [§4.3, §3.1]
 *   2. every Context block scored against the current query                          [§3.1, §4.3]
 *   3. the top-k Context blocks selected, per KV head or shared by all KV heads      [§4.5]
 *   4. exact softmax attention over Initial blocks + selected blocks + Local window  [§4.2, §4.6]
 * Knob names follow the article's configuration list [§4.5] and the operator constructor on
 * "How to Implement Long Context Inference (Up to 139K Tokens) with KTransformers" (instagit),
 * step 3: block_size, local_windows_len, topk/second_select_num, anchor_type, anchor_num,
 * head_select_mode.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked "host".  The caller owns all memory; the library
 *     never allocates, frees or synchronises.  What carries over between calls is (a) the
 *     hand-off counters inside a kvs_decode_step workspace (see there: such a workspace belongs to
 *     kvs_decode_step alone), (b) the per-thread text behind kvs_last_error and (c) the static
 *     device scratch area of kvs_decode_step_noalloc (one per GPU, see there).  Calls from several
 *     host threads are safe when they use distinct workspaces and outputs.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null stream).
 *   - Every argument that can be checked on the host is checked before anything is enqueued; on
 *     error the call returns a negative status and enqueues nothing.  Contents of device buffers
 *     (sequence lengths, table entries, selections) are the caller's responsibility: out-of-range
 *     values there are undefined behaviour.
 *   - Debug mode: with the environment variable KVS_DEBUG set (and not "0") when a call is made,
 *     every entry point that reads such contents first waits for `stream`, copies them to the host
 *     and checks them as kvs_validate_contents does (block ids of kvs_build_reps /
 *     kvs_quantize_kv: >= 0); bad contents return KVS_ERR_INVALID_ARG, with the first bad entry in
 *     kvs_last_error, and nothing is enqueued.  The check is skipped while the stream is being
 *     captured into a graph.  This mode synchronises; results are otherwise unchanged.
 *   - v1 limits: head_dim == 128, block_size == 128, num_kv_heads in {1,2,4,8,16},
 *     num_q_heads / num_kv_heads in {1,2,4,8,16}.  Other shapes return KVS_ERR_UNSUPPORTED.
 *
 * Layouts (row-major, innermost last)
 *   q            fp16 [batch][Hq][128]
 *   out          fp32 [batch][Hq][128]
 *   k_pool,v_pool kv_type FP16: fp16 [n_phys][Hkv][128 tokens][128], one (block, KV head) tile = 32 KiB
 *                kv_type Q8_0: [n_phys][Hkv] records of 17408 bytes, one per (block, KV head):
 *                int8 codes [128 tokens][128], then fp16 scales [128 tokens][4]; channel c of token
 *                t holds scale[t][c / 32] * code[t][c] (see kvs_quantize_kv)
 *                kv_type Q4_0: [n_phys][Hkv] records of 9216 bytes: codes [128 tokens][64 bytes], word k
 *                of a row holding channels 8k..8k+7 (channel 8k+2i in bits 4i..4i+3, 8k+2i+1 in bits
 *                16+4i..19+4i), then fp16 scales [128 tokens][4]; value scale * (code - 8)
 *                kv_type INT8_PTH: [n_phys][Hkv] records of 16896 bytes: int8 codes [128 tokens][128],
 *                then fp32 scales [128 tokens]; value fp32(scale[t] * code[t][c])
 *                kv_type INT4_PTH: [n_phys][Hkv] records of 8832 bytes: codes as Q4_0's, then fp32
 *                scales [128 tokens], then uint8 zero points [128 tokens]; value
 *                fp32(scale[t] * (code[t][c] - zero[t]))
 *   rep_pool     [n_phys][Hkv][R][128]  fp16, except fp32 for KVS_REP_MEAN.
 *                R = 2 for Quest (r=0 channel-wise min key, r=1 channel-wise max key), 1 for Max
 *                and Mean, rep_num for Fix (r-th rep = token r*(128/rep_num) of the block).
 *   block_table  int32 [batch][max_blocks_per_seq]: logical block -> physical block id
 *   seq_lens     int32 [batch]: cached tokens per sequence, the current token included (>= 1)
 *   scores       fp32 [batch][G][max_blocks_per_seq], G = Hkv (SEPARATE) or 1 (SHARED);
 *                -INFINITY at every non-candidate block
 *   sel          int32 [batch][G][topk]: selected logical block ids in ascending order, -1 padded
 *   sel_count    int32 [batch][G]
 *   Query head j reads KV head j / (Hq/Hkv) (contiguous GQA groups).
 *   q, the pools and rep_pool must be 16-byte aligned (KVS_ERR_MISALIGNED otherwise).
 *
 * Regions of a sequence of L tokens (block size B, lengths rounded outward to whole blocks):
 *   I_b   = B * ceil(initial_len / B)                         Initial = [0, min(I_b, L))
 *   L_loc = max(I_b, B * floor((L - local_len) / B))          Local   = [L_loc, L)
 *   candidates = logical blocks b with I_b <= b*B and (b+1)*B <= L_loc; none if L <= I_b.
 *   k_eff = min(topk, number of candidates).
 */
#ifndef KVS_H
#define KVS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* kvs_stream_t; /* hipStream_t */

enum {
  KVS_OK = 0,
  KVS_ERR_INVALID_ARG = -1, /* null pointer, negative size, inconsistent shapes     */
  KVS_ERR_UNSUPPORTED = -2, /* a shape outside the v1 limits above                  */
  KVS_ERR_MISALIGNED = -3,  /* q / pools / rep_pool not 16-byte aligned             */
  KVS_ERR_WORKSPACE = -4,   /* workspace null or smaller than the size query        */
  KVS_ERR_HIP = -5          /* a kernel launch failed                               */
};

/* Rep methods [KT-LC §4.3].  Dynamic reps are built from token scores (kvs_token_importance,
 * kvs_build_dynamic_reps) and scored like Fix. */
typedef enum { KVS_REP_QUEST = 0, KVS_REP_MAX = 1, KVS_REP_MEAN = 2, KVS_REP_FIX = 3,
               KVS_REP_DYNAMIC = 4 } kvs_rep_method;

/* head_select_mode [KT-LC §4.5]: SEPARATE = every KV head selects its own blocks from the scores
 * of its query heads (summed); SHARED = one selection for all heads from the sum over all
 * query heads. */
typedef enum { KVS_HEADS_SEPARATE = 0, KVS_HEADS_SHARED = 1 } kvs_head_select_mode;

/* Cache precision of k_pool / v_pool: the operator's kv_type [KT-LC §4.5 configuration list; the
 * instagit page's operator constructor, step 3], which names FP16, FP32, Q4_0 and Q8_0.  FP16, Q8_0
 * and Q4_0 are provided, the last two being llama.cpp's published block formats, per token and KV head
 * in blocks of 32 channels with an fp16 scale:
 *   Q8_0: d = max|x| / 127, int8 codes round(x / d) ties away from zero, value d * code;
 *   Q4_0: m = the first value of largest magnitude, d = m / -8, codes min(15, trunc(x / d + 8.5)) in
 *         0..15, value d * (code - 8).
 * INT8_PTH is the int8 cache with one dynamic scale per token and head of the page "Long context:
 * 262k with KVarN, and the built-in KV modes" (section "The built-in per-token-head modes"), with
 * Q8_0's arithmetic over a whole 128-channel row:
 *   s = max|x| / 127 kept in fp32, codes round(x / s) ties away from zero, value fp32(s * code).
 * INT4_PTH is that page's int4 per-token-head cache (dynamic scales with asymmetric zero points; its
 * rotation is not defined there and not applied), read as asymmetric quantization per token's row:
 *   lo = min(0, min x), hi = max(0, max x), s = (hi - lo) / 15 kept in fp32, z = rint(-lo / s) in
 *   0..15 kept as a byte, codes clamp(rint(x / s) + z, 0, 15), rint to even, value fp32(s * (code - z)). */
typedef enum {
  KVS_KV_FP16 = 0, KVS_KV_Q8_0 = 1, KVS_KV_Q4_0 = 2, KVS_KV_INT8_PTH = 3, KVS_KV_INT4_PTH = 4
} kvs_kv_type;

/* Host struct.  Field order and types are part of the ABI. */
typedef struct kvs_config {
  int32_t num_q_heads;      /* Hq                                                           */
  int32_t num_kv_heads;     /* Hkv, Hq % Hkv == 0                                            */
  int32_t head_dim;         /* d, must be 128                                                */
  int32_t block_size;       /* B tokens per block, must be 128 [KT-LC §4.3, §5.1]            */
  int32_t initial_len;      /* Initial tokens, >= 0 [KT-LC §4.2]                             */
  int32_t local_len;        /* local_windows_len, >= 0 [KT-LC §4.2, §4.5]                    */
  int32_t topk;             /* second_block_count: Context blocks selected, >= 0 [KT-LC §4.5] */
  int32_t rep_method;       /* kvs_rep_method (anchor_type)                                  */
  int32_t rep_num;          /* anchor_num: Fix (divides B) and Dynamic, 1..B; ignored otherwise */
  int32_t head_select_mode; /* kvs_head_select_mode                                          */
  float softmax_scale;      /* attention logit scale; 0 => 1/sqrt(head_dim) [KT-LC §4.6]     */
  int32_t kv_type;          /* kvs_kv_type of k_pool and v_pool                              */
} kvs_config;

/* Human-readable name of a status code (static string). */
const char* kvs_status_string(int status);

/* Detail of the last failed call on the calling thread (for KVS_ERR_HIP: the HIP error name and
 * message and the launch that failed); "" if no call on this thread has failed.  The string stays
 * valid until the next failing call on the same thread. */
const char* kvs_last_error(void);

/*
 * kvs_validate_contents -- the device-content rules of the entry points, checked on HOST copies
 * (what KVS_DEBUG=1 runs before each call).  All pointers are host pointers; block_table, sel /
 * sel_count and presel are nullable (not checked when null).  Rules, per sequence i:
 *   1 <= seq_lens[i] <= max_blocks_per_seq * 128;
 *   block_table[i][b] >= 0 for every block b the sequence uses (b < ceil(seq_lens[i] / 128));
 *   per group gr: 0 <= sel_count[i][gr] <= min(topk, candidates at seq_lens[i]); the first
 *   sel_count entries of sel[i][gr] are distinct candidate blocks of the current length (what an
 *   older selection of the same sequence still satisfies: candidates only grow);
 *   presel[i][gr][e] in [-1, max_blocks_per_seq).
 * Returns KVS_OK, or KVS_ERR_INVALID_ARG with the first bad entry described in kvs_last_error.
 * The upper bound of physical ids is not checked: the pools' sizes are not arguments.
 */
int kvs_validate_contents(const kvs_config* cfg, const int32_t* seq_lens, int32_t batch,
                          const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* sel,
                          const int32_t* sel_count, const int32_t* presel, int32_t n_presel);

/* Reps per (block, KV head) for this config, or a negative status. */
int kvs_rep_count(const kvs_config* cfg /* host */);

/* Bytes of one physical block's reps over all KV heads (Hkv * R * 128 * elem), 0 on bad config. */
size_t kvs_rep_bytes_per_block(const kvs_config* cfg /* host */);

/* Bytes of one physical block of k_pool (or v_pool) over all KV heads: Hkv * 32768 for FP16,
 * Hkv * 17408 for Q8_0, Hkv * 9216 for Q4_0, Hkv * 16896 for INT8_PTH, Hkv * 8832 for INT4_PTH;
 * 0 on a bad config. */
size_t kvs_kv_bytes_per_block(const kvs_config* cfg /* host */);

/*
 * kvs_quantize_kv -- Q8_0 / Q4_0 / INT8_PTH / INT4_PTH records of fp16 tiles [kv_type, see kvs_kv_type].  For each of
 * the n_blocks physical ids in phys_block_ids (device int32) and each KV head, reads the fp16 tile
 * [128 tokens][128] of src_pool (laid out as an FP16 pool) and writes the record at the same id of
 * dst_pool (laid out as a pool of cfg->kv_type).  Per 32 channels of a token, in fp32 with IEEE
 * division: Q8_0 d = max|x| / 127, codes round(x * (1/d)) ties away from zero (an all-zero block:
 * d = 0, codes 0); Q4_0 d = m / -8 for m the first value of largest magnitude (+0 for an all-zero
 * block), codes min(15, trunc(x * (1/d) + 8.5)) (all-zero: 8).  d is stored rounded to fp16.
 * INT8_PTH: per token, s = max|x| / 127 over its 128 channels, codes as Q8_0's, s stored as fp32.
 * INT4_PTH: per token, lo = min(0, min x), hi = max(0, max x), s = (hi - lo) / 15, inv = 1 / s,
 * z = clamp(rint(-lo * inv), 0, 15), codes clamp(rint(x * inv) + z, 0, 15), rint to even (an all-zero
 * row: s = 0, z = 0, codes 0); s stored as fp32, z as a byte.
 * Used for keys and values alike.  cfg->kv_type must be Q8_0, Q4_0, INT8_PTH or INT4_PTH.
 * n_blocks == 0 is a no-op.  Both pools 16-byte aligned.
 */
int kvs_quantize_kv(const kvs_config* cfg, const void* src_pool, const int32_t* phys_block_ids,
                    int32_t n_blocks, void* dst_pool, kvs_stream_t stream);

/*
 * kvs_build_reps -- representative keys of full blocks [KT-LC §4.3; Quest's "Reduced Keys" §3.1].
 * For each of the n_blocks physical ids in phys_block_ids (device int32) and each KV head, reads
 * the 128x128 key tile and writes its reps into rep_pool at the same physical id:
 *   Quest: channel-wise min (r=0) and max (r=1);  Max: channel-wise max;
 *   Mean:  channel-wise mean in fp32;             Fix: rows 0, s, 2s, ... with s = 128/rep_num.
 * Every listed block must be full (128 valid tokens).  n_blocks == 0 is a no-op.  Dynamic reps come
 * from kvs_build_dynamic_reps instead (KVS_ERR_INVALID_ARG here).
 * With a quantized kv_type the reps are taken over the cached values (fp32) and stored rounded to
 * fp16 (Mean: fp32).
 */
int kvs_build_reps(const kvs_config* cfg, const void* k_pool, const int32_t* phys_block_ids,
                   int32_t n_blocks, void* rep_pool, kvs_stream_t stream);

/* Workspace bytes kvs_token_importance needs (host query; 0 on bad config or sizes). */
size_t kvs_importance_workspace_size(const kvs_config* cfg, int32_t batch, int32_t max_blocks_per_seq,
                                     int32_t n_obs);

/*
 * kvs_token_importance -- cumulative attention score of every cached token, the input of Dynamic
 * reps [KT-LC §4.3 rep table: Dynamic takes the tokens of a block with the highest accumulated
 * attention score; the scoring method is left open there and is this one].  q_obs: fp16
 * [batch][n_obs][Hq][128], the queries of each sequence's last n_obs cached tokens (positions
 * L-n_obs .. L-1, in order; 1 <= n_obs <= L and n_obs <= 4096).  importance: fp32
 * [batch][G][max_blocks_per_seq * 128]; for token t of a sequence and group gr (SEPARATE: KV head;
 * SHARED: 0):
 *   importance = sum over observation queries i and the group's query heads j of
 *                softmax_t'(scale * q_ij . K[t']) at t' = t, over the keys t' <= L - n_obs + i,
 * zero for t >= L.  Accumulation fp32.  With a quantized kv_type the keys are the cached values (the
 * codes times their scales, applied in fp32).
 * workspace: device, >= kvs_importance_workspace_size bytes, 256-byte aligned, scratch.
 */
int kvs_token_importance(const kvs_config* cfg, const void* q_obs, int32_t n_obs, const void* k_pool,
                         const int32_t* block_table, int32_t max_blocks_per_seq,
                         const int32_t* seq_lens, int32_t batch, float* importance, void* workspace,
                         size_t workspace_bytes, kvs_stream_t stream);

/*
 * kvs_build_dynamic_reps -- Dynamic reps [KT-LC §4.3].  For every full block b of every sequence
 * (b*128 + 128 <= L) and every KV head h: the K rows of the rep_num tokens of the block with the
 * highest importance (group of h; ties to the lower token), in ascending token order, written to
 * rep_pool at the block's physical id.  cfg->rep_method must be KVS_REP_DYNAMIC.  With a quantized
 * kv_type the reps are those rows' cached values rounded to fp16.
 */
int kvs_build_dynamic_reps(const kvs_config* cfg, const void* k_pool, const float* importance,
                           const int32_t* block_table, int32_t max_blocks_per_seq,
                           const int32_t* seq_lens, int32_t batch, void* rep_pool,
                           kvs_stream_t stream);

/* Workspace bytes kvs_preselect_blocks needs (host query; 0 on bad config or sizes). */
size_t kvs_preselect_workspace_size(const kvs_config* cfg, int32_t batch, int32_t max_blocks_per_seq);

/*
 * kvs_preselect_blocks -- the preselected set [KT-LC §4.4 Preselect, after SnapKV; §4.5
 * preselect_block_count; §4.6 preselect_block]: before decoding, the blocks the question's tokens
 * attend most.  Per (sequence, group), each candidate block gets a preselect score from importance
 * (kvs_token_importance; same groups; 16-byte aligned):
 *   pool_kernel == 0: the sum of its 128 token scores;
 *   pool_kernel odd, 1..127: its largest pooled vote, a token's pooled vote being the mean of the
 *     Context token scores in the window of pool_kernel tokens centred on it (tokens outside the
 *     Context count as zero; the divisor is always pool_kernel).  Ranking blocks so is the same as
 *     taking tokens in descending pooled vote until n_presel distinct blocks are hit.
 * The min(n_presel, candidates) best blocks, ties to the lower block, are written ascending to
 * presel [batch][G][n_presel], -1 padded, with their number in presel_count [batch][G].
 * workspace: >= kvs_preselect_workspace_size bytes, 256-byte aligned.  Any other pool_kernel:
 * KVS_ERR_INVALID_ARG.
 */
int kvs_preselect_blocks(const kvs_config* cfg, const float* importance, const int32_t* seq_lens,
                         int32_t batch, int32_t max_blocks_per_seq, int32_t n_presel,
                         int32_t pool_kernel, int32_t* presel,
                         int32_t* presel_count, void* workspace, size_t workspace_bytes,
                         kvs_stream_t stream);

/* Workspace bytes kvs_decode_step_preselected needs (host query; 0 on bad config or sizes). */
size_t kvs_decode_step_preselected_workspace_size(const kvs_config* cfg, int32_t batch,
                                                  int32_t max_blocks_per_seq, int32_t n_presel);

/*
 * kvs_decode_step_preselected -- kvs_decode_step with every selection confined to a preselected set
 * [KT-LC §4.4]: per (sequence, group), only the blocks of presel [batch][G][n_presel] (ascending, -1
 * padded, e.g. from kvs_preselect_blocks) that are still candidates at the current length compete;
 * k_eff = min(topk, their number), so with topk >= the set's size the set is attended as it is.
 * Scores, ties, order and attention as kvs_decode_step.  With topk > 0, n_presel <= 1024 and
 * batch * G <= 16384, enqueued as three launches: 1. scoring of the sets' blocks only (with some of
 * the Initial/Local tiles);  2. attention over the selected tiles, where the workgroup of each selected
 * tile makes its (sequence, group)'s selection from the scored set itself, and over the other
 * Initial/Local tiles (for batch * num_kv_heads * topk <= 1024; otherwise the selection is made in
 * launch 1 by the scoring workgroup of the (sequence, group) that finishes last, with every
 * Initial/Local tile);  3. the merge.  Otherwise: scoring of
 * every candidate (with the Initial/Local tiles for max_blocks_per_seq <= 2048), a ranking of the
 * set (n_presel <= 256) or compaction, top-k and mapping, attention tiles and merge.
 * workspace: >= the size query, 256-byte aligned.  Like kvs_decode_step's, its first 64 KiB hold
 * hand-off counters: zero-fill it once before its first use; every call that runs to completion
 * leaves them zero, a call that did not complete may not, and the workspace must then be zeroed
 * again.  It belongs to this entry point alone (another call writing into it breaks the counters).
 * sel_out / sel_count_out (nullable) receive the selection.
 */
int kvs_decode_step_preselected(const kvs_config* cfg, const void* q, const void* k_pool,
                                const void* v_pool, const void* rep_pool, const int32_t* block_table,
                                int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                                const int32_t* presel, int32_t n_presel, float* out, int32_t* sel_out,
                                int32_t* sel_count_out, void* workspace, size_t workspace_bytes,
                                kvs_stream_t stream);

/*
 * kvs_score_blocks -- block relevance [KT-LC §3.1 Quest bound; §4.3 rep similarity; §4.5 modes].
 * For every candidate block b of every sequence and query head j (KV head h = j/g):
 *   Quest:        s_j(b) = sum_c max(q_jc * kmax_hbc, q_jc * kmin_hbc)
 *   Max/Mean/Fix/Dynamic: s_j(b) = sum_r sum_c q_jc * rep_hbrc
 * (no softmax scale), then SEPARATE: scores[h][b] = sum of s_j over the query heads of h;
 * SHARED: scores[0][b] = sum over all query heads.  Non-candidates get -INFINITY.
 * Accumulation is fp32.
 */
int kvs_score_blocks(const kvs_config* cfg, const void* q, const void* rep_pool,
                     const int32_t* block_table, int32_t max_blocks_per_seq,
                     const int32_t* seq_lens, int32_t batch, float* scores, kvs_stream_t stream);

/*
 * kvs_topk_blocks -- top-k selection [KT-LC §3.1 "top-k blocks"; §4.5 second_block_count].
 * Per (sequence, group): the k_eff best candidates by score, ties to the lower block index, written
 * to sel in ascending block order and padded with -1; sel_count = k_eff.  NaN scores are undefined.
 */
int kvs_topk_blocks(const kvs_config* cfg, const float* scores, const int32_t* seq_lens,
                    int32_t batch, int32_t max_blocks_per_seq, int32_t* sel, int32_t* sel_count,
                    kvs_stream_t stream);

/* Workspace bytes kvs_sparse_decode_attn needs for these sizes (host query; 0 on bad config). */
size_t kvs_attn_workspace_size(const kvs_config* cfg, int32_t batch, int32_t max_blocks_per_seq);

/*
 * kvs_sparse_decode_attn -- exact attention over the retrieved cache [KT-LC §4.2, §4.6].
 * For query head j of sequence i (group = its KV head in SEPARATE mode, 0 in SHARED):
 *   T = Initial tokens + every token of the sel_count selected blocks + Local tokens
 *   out[i][j] = sum_{t in T} softmax_t(scale * q_j . K[t]) V[t], accumulated in fp32.
 * sel may come from an earlier step (re-selection every token_step tokens / layer_step layers,
 * [KT-LC §4.6]): Local only grows, so an old selection still names Context blocks.  Selected ids
 * must be candidates of the current length and distinct.  workspace: device, at least
 * kvs_attn_workspace_size bytes, 256-byte aligned; its contents are scratch.
 */
int kvs_sparse_decode_attn(const kvs_config* cfg, const void* q, const void* k_pool,
                           const void* v_pool, const int32_t* block_table,
                           int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch,
                           const int32_t* sel, const int32_t* sel_count, float* out,
                           void* workspace, size_t workspace_bytes, kvs_stream_t stream);

/* Workspace bytes kvs_decode_step needs (host query; 0 on bad config). */
size_t kvs_decode_step_workspace_size(const kvs_config* cfg, int32_t batch,
                                      int32_t max_blocks_per_seq);

/*
 * kvs_decode_step -- one decode step of one layer: score -> top-k -> sparse attention
 * [KT-LC §4.6, retrieval then attention], enqueued with no host synchronisation as
 *   for max_blocks_per_seq <= 2048 and batch * num_kv_heads * topk <= 1024, three launches:
 *   1. scoring (with some of the Initial/Local tiles' attention: they do not depend on the
 *   selection);  2. attention over the selected tiles, where the workgroup of each selected tile
 *   makes its (sequence, group)'s top-k itself from the scores (every one of them the same), and
 *   over the other Initial/Local tiles;  3. the log-sum-exp merge into out;
 *   for other max_blocks_per_seq <= 2048, three launches: 1. scoring, top-k per (sequence, group) by
 *   the scoring workgroup of the group that finishes last, and the Initial/Local tiles' attention;
 *   2. attention over the selected tiles;  3. the merge;
 *   SEPARATE with 2048 < max_blocks_per_seq <= 16384 and topk > 0, three launches in which each
 *   scoring workgroup (64 blocks of one KV head) also stores its 8 best blocks and the selection is
 *   made from these summaries -- for batch * num_kv_heads * topk <= 1024 by the workgroup of each
 *   selected tile (1. scoring;  2. the selected tiles, each making its KV head's top-k, and the
 *   Initial/Local tiles;  3. the merge), otherwise by the last scoring workgroup of the KV head, in
 *   the scoring launch with the Initial/Local tiles; when a chunk of 64 blocks holds more than 8 of
 *   the selection (the summaries cannot tell which), it is made from the whole score row instead;
 *   otherwise four: 1. scoring;  2. top-k, with the Initial/Local tiles' attention;  3. attention
 *   over the selected tiles;  4. the merge.
 * Top-k also resolves the selected blocks' physical ids.
 * Results equal kvs_score_blocks + kvs_topk_blocks + kvs_sparse_decode_attn on the same inputs.
 * Reps must be current for every candidate block (kvs_build_reps).  sel_out / sel_count_out
 * (nullable) receive the selection for reuse by later kvs_sparse_decode_attn calls.
 * workspace: device, >= kvs_decode_step_workspace_size bytes, 256-byte aligned.  Its first 64 KiB
 * hold hand-off counters: zero-fill the workspace once before its first use (e.g. hipMemset); every
 * call that runs to completion leaves the counters zero again, so the workspace can then be reused
 * by later kvs_decode_step calls, of any config and size that fits.  Such a workspace belongs to
 * kvs_decode_step alone: the other entry points write their own data from offset 0 and would leave
 * non-zero counters, and so would a call that did not complete (a failed launch, an aborted
 * stream); zero-fill it again after either.  Counters that are not zero leave the selection
 * unmade and the attention reading stale tile ids.  The rest is scratch.  Calls sharing one
 * workspace must not run concurrently (stream order is enough).  batch * G must not exceed 16384
 * (KVS_ERR_UNSUPPORTED).
 */
int kvs_decode_step(const kvs_config* cfg, const void* q, const void* k_pool, const void* v_pool,
                    const void* rep_pool, const int32_t* block_table, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, int32_t batch, float* out, int32_t* sel_out,
                    int32_t* sel_count_out, void* workspace, size_t workspace_bytes,
                    kvs_stream_t stream);

/*
 * kvs_decode_step_noalloc -- kvs_decode_step for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid allocation): the same kernels and
 * results, with the workspace taken from a static device scratch area of KVS_NOALLOC_SCRATCH_BYTES
 * that every GPU the library runs on holds until the process ends.  No allocation is made by this
 * call or by the library.  The first call on a device looks the area up and enqueues one small
 * kernel on `stream` that clears its hand-off counters; every completed call leaves them zero.
 * Sizes whose kvs_decode_step_workspace_size exceeds KVS_NOALLOC_SCRATCH_BYTES return
 * KVS_ERR_WORKSPACE (the needed size in kvs_last_error) and enqueue nothing.  All calls on one
 * device share its scratch: calls that may overlap on one GPU (other streams, other host threads)
 * race and must be ordered by the caller.  Other arguments and errors as kvs_decode_step.
 */
#define KVS_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int kvs_decode_step_noalloc(const kvs_config* cfg, const void* q, const void* k_pool, const void* v_pool,
                            const void* rep_pool, const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, int32_t batch, float* out, int32_t* sel_out,
                            int32_t* sel_count_out, kvs_stream_t stream);

/*
 * kvs_gather_read_floor -- a measurement, not a step of the method: how long this device takes to
 * read K/V tiles of the fp16 pools with nothing else done, for comparison with the attention
 * launches that read the same tiles.  Workgroup x (256 lanes) reads the K tile and the V tile
 * tile_ids[x] = phys_block * num_kv_heads + kv_head (128 tokens x 128 channels of fp16 each,
 * contiguous in its pool), every 16-byte load of a lane issued before any is used, and writes the
 * fp32 sum of the tile's 32,768 values to out[x].  lds_bytes (0 to 65,536) of LDS is reserved per
 * workgroup and not used: it sets how many workgroups share a CU (an attention tile's workgroup
 * reserves 36,864 bytes).  pool_tiles: the tiles each pool holds (phys blocks x num_kv_heads);
 * tile_ids: device, n_tiles entries; an entry outside [0, pool_tiles) reads nothing and gives
 * out[x] = NaN.  out: device, n_tiles floats.  n_tiles == 0 enqueues nothing.
 */
int kvs_gather_read_floor(const void* k_pool, const void* v_pool, int32_t pool_tiles,
                          const int32_t* tile_ids, int32_t n_tiles, int32_t lds_bytes, float* out,
                          kvs_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* KVS_H */
