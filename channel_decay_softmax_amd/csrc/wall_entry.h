// wall_entry.h -- checks and launches shared by more than one entry point of
// the C ABI (library-internal).
#pragma once

#include "wall.h"

namespace wall {

// The argument checks of wall_attn_decode other than its workspace.
wall_status_t decode_check(const void *q, const void *v, wall_dtype_t dtype, const float *p_curr,
                           int64_t p_curr_batch_stride, const void *k_tilde, const float *r_cache,
                           const float *sink_bias, const void *o, const float *lse, int64_t B, int64_t T,
                           int64_t T_cap, int64_t HQ, int64_t H, int64_t K, int64_t V, int64_t chunk_size);
// The decode launches on checked arguments, with `part` (at least
// decode_layout(B, T, HQ, V).total bytes of device memory) for the split
// partials.
wall_status_t decode_launch(const void *q, const void *v, wall_dtype_t dtype, const float *p_curr,
                            int64_t p_curr_batch_stride, const void *k_tilde, const float *r_cache,
                            const float *sink_bias, void *o, float *lse, int64_t B, int64_t T, int64_t T_cap,
                            int64_t HQ, int64_t H, int64_t K, int64_t V, int64_t chunk_size, float scale,
                            float *part, hipStream_t stream);

}  // namespace wall
