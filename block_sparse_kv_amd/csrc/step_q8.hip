// The decode step's kernels for kv_type Q8 (step_body.h).
#include "step_body.h"

namespace kvs {
template hipError_t launch_score_select_kv<kKvQ8>(const AttnArgs&, const void*, float*, int32_t*, int32_t*,
                                                int32_t*, int*, int, hipStream_t,
                                                const Summaries&, int);
template hipError_t launch_attn_select_kv<kKvQ8>(const AttnArgs&, const float*, int32_t*, int32_t*, int,
                                               int, hipStream_t, const Summaries&, int);
template hipError_t launch_topk_il_wide_kv<kKvQ8>(const AttnArgs&, const float*, int32_t*, int32_t*, int32_t*,
                                                int, hipStream_t);
template hipError_t launch_presel_step_kv<kKvQ8>(const AttnArgs&, const void*, const int32_t*, int, float*,
                                                int32_t*, int32_t*, int32_t*, int32_t*, int*, int,
                                                hipStream_t, int);
}  // namespace kvs
