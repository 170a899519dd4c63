// Host-side pieces of the C ABI shared between api.cpp and the allocation-free
// entry point (noalloc.hip).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "csa.h"

namespace csa_api {

// Record an error detail for csa_last_error() and return the status.
csa_status fail(csa_status s, const char *fmt, ...);

// Per-row scales of fp8 (E4M3) index tensors (csa_attention_fp8).
struct IndexFp8 {
    const float *q_scale;        // [B*T, HI]
    const void *const *k_scale;  // [B] -> [N_b] float
};

// The fused CSA step (csa_attention, or csa_attention_fp8 when f8 is given:
// q_idx and k_idx then hold E4M3 codes) on the device work area ws of ws_bytes
// bytes: every argument check, then the launches on `stream`.
csa_status attention_impl(const csa_dims *d, const void *q, const void *q_idx, const float *w,
                          const void *const *k_idx, const void *const *kv, const void *const *v,
                          const void *const *win, const void *const *win_v, const int32_t *win_pos0,
                          const int32_t *win_rows, const int32_t *seq_len, const int32_t *q_pos, const float *sink,
                          float *out, float *lse, int32_t *topk_idx_out, float *scores_out, void *ws,
                          size_t ws_bytes, void *stream, const IndexFp8 *f8 = nullptr);

}  // namespace csa_api
