// C ABI of libcsa: argument checks (host only, before any enqueue), workspace
// sizing and the launch chain.  Declarations and contracts are in csa.h.
#include "csa.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "api_internal.hpp"
#include "launch.hpp"

namespace {
thread_local std::string g_last_error;
}  // namespace

namespace csa_api {
csa_status fail(csa_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}
}  // namespace csa_api

namespace {
using csa_api::fail;

csa_status ok() {
    g_last_error.clear();
    return CSA_OK;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

#define REQUIRE_PTR(p)                                                      \
    do {                                                                    \
        if (!(p)) return fail(CSA_ERR_NULL, "argument '%s' is NULL", #p);   \
    } while (0)
#define REQUIRE_ALIGN(p, a)                                                                   \
    do {                                                                                      \
        if ((p) && !aligned((p), (a)))                                                        \
            return fail(CSA_ERR_ALIGN, "argument '%s' is not %d-byte aligned", #p, (int)(a)); \
    } while (0)

constexpr int kMaxQueries = 1 << 20;
constexpr int kMaxEntries = 1 << 26;

int n_queries(const csa_dims *d) { return d->batch * d->q_len; }

csa_status check_common(const csa_dims *d) {
    if (!d) return fail(CSA_ERR_NULL, "argument 'dims' is NULL");
    if (d->batch <= 0 || d->q_len <= 0) return fail(CSA_ERR_DIM, "batch and q_len must be >= 1");
    if ((long long)d->batch * d->q_len > kMaxQueries)
        return fail(CSA_ERR_DIM, "batch * q_len exceeds %d", kMaxQueries);
    if (d->ratio < 1) return fail(CSA_ERR_DIM, "ratio must be >= 1");
    if (d->max_entries < 1 || d->max_entries > kMaxEntries)
        return fail(CSA_ERR_DIM, "max_entries must be in [1, %d]", kMaxEntries);
    if (d->dtype != CSA_F32 && d->dtype != CSA_BF16) return fail(CSA_ERR_UNSUPPORTED, "unknown dtype %d", d->dtype);
    return CSA_OK;
}

csa_status check_scores(const csa_dims *d) {
    if (d->index_heads <= 0 || d->index_dim <= 0) return fail(CSA_ERR_DIM, "index_heads and index_dim must be >= 1");
    if (d->index_act != CSA_ACT_RELU && d->index_act != CSA_ACT_NONE)
        return fail(CSA_ERR_UNSUPPORTED, "unknown index_act %d", d->index_act);
    if (d->dtype == CSA_BF16 && (d->index_heads != 64 || d->index_dim != 128))
        return fail(CSA_ERR_UNSUPPORTED, "bf16 scorer needs index_heads 64 and index_dim 128 (got %d, %d)",
                    d->index_heads, d->index_dim);
    if (d->dtype == CSA_F32 && (d->index_heads > 64 || d->index_dim > 128))
        return fail(CSA_ERR_UNSUPPORTED, "fp32 scorer supports index_heads <= 64, index_dim <= 128");
    return CSA_OK;
}

// fp8 index tensors: the decode scorer's shape (64 heads x 128 dims)
csa_status check_scores_fp8(const csa_dims *d) {
    if (d->index_act != CSA_ACT_RELU && d->index_act != CSA_ACT_NONE)
        return fail(CSA_ERR_UNSUPPORTED, "unknown index_act %d", d->index_act);
    if (d->index_heads != 64 || d->index_dim != 128)
        return fail(CSA_ERR_UNSUPPORTED, "fp8 scorer needs index_heads 64 and index_dim 128 (got %d, %d)",
                    d->index_heads, d->index_dim);
    return CSA_OK;
}

csa_status check_topk(const csa_dims *d) {
    if (d->topk < 1 || d->topk > csa::kTopkMaxK) return fail(CSA_ERR_DIM, "topk must be in [1, %d]", csa::kTopkMaxK);
    return CSA_OK;
}

csa_status check_attn(const csa_dims *d) {
    if (d->n_heads <= 0 || d->head_dim <= 0) return fail(CSA_ERR_DIM, "n_heads and head_dim must be >= 1");
    if (d->window < 1) return fail(CSA_ERR_DIM, "window must be >= 1");
    if (!(d->softmax_scale >= 0.f) || !std::isfinite(d->softmax_scale))
        return fail(CSA_ERR_DIM, "softmax_scale must be finite and >= 0");
    if (d->dtype == CSA_BF16 && ((d->n_heads != 64 && d->n_heads != 128) || d->head_dim != 512))
        return fail(CSA_ERR_UNSUPPORTED, "bf16 attention needs n_heads 64 or 128 and head_dim 512 (got %d, %d)",
                    d->n_heads, d->head_dim);
    if (d->dtype == CSA_F32 && (d->n_heads > 128 || d->head_dim > 512))
        return fail(CSA_ERR_UNSUPPORTED, "fp32 attention supports n_heads <= 128, head_dim <= 512");
    if (d->dtype == CSA_BF16 && (long long)d->max_entries + d->window > (1ll << 28))
        return fail(CSA_ERR_DIM, "too many rows per query");
    return CSA_OK;
}

float scale_of(const csa_dims *d) {
    return d->softmax_scale > 0.f ? d->softmax_scale : 1.f / std::sqrt((float)d->head_dim);
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// Histogram windows come from the bf16 or fp8 scorer in the fused call (one per
// decode-scorer workgroup, or per entry chunk of the tiled bf16 scorer) and
// from the top-k's own histogram kernel otherwise (0 here).  The fp8 index
// path always takes the decode scorer.
// The decode scorer's geometry in the fused call (the tiled bf16 scorer for many
// queries per sequence has none): windows and regions per query, emitted
// entries per region.
bool fused_decode(const csa_dims *d, bool fp8) {
    return d->dtype == CSA_BF16 && (fp8 || !csa::score_uses_tiles(csa::kBF16, d->q_len));
}
csa::DecodeGeom decode_geom(const csa_dims *d, bool fp8) {
    return csa::decode_geom(fp8, d->max_entries, n_queries(d), d->topk);
}
int win_count(const csa_dims *d, bool fused, bool fp8 = false) {
    if (!fused || d->dtype != CSA_BF16) return 0;
    if (!fused_decode(d, fp8)) return csa::tiled_windows(d->batch, d->q_len, d->max_entries);
    return decode_geom(d, fp8).n_win;
}
// Entries per scorer region (a decode-scorer workgroup, or a (query, entry
// chunk) of the tiled scorer) handed to the selection in the fused call (0: the
// selection scans the scores itself).
int emit_cap(const csa_dims *d, bool fused, bool fp8 = false) {
    if (!fused || d->dtype != CSA_BF16 || !csa::topk_uses_histogram(d->max_entries)) return 0;
    if (!fused_decode(d, fp8)) return csa::tiled_emit_cap(d->batch, d->q_len, d->max_entries, d->topk);
    return decode_geom(d, fp8).em_cap;
}
size_t ws_topk(const csa_dims *d, bool fused = false, bool fp8 = false) {
    return csa::topk_workspace_bytes(n_queries(d), d->topk, d->max_entries, win_count(d, fused, fp8),
                                     emit_cap(d, fused, fp8));
}
size_t ws_sparse(const csa_dims *d) {
    return csa::mqa_workspace_bytes(d->dtype, n_queries(d), d->n_heads, d->head_dim, d->topk + d->window);
}
size_t ws_hca(const csa_dims *d) {
    return csa::mqa_workspace_bytes(d->dtype, n_queries(d), d->n_heads, d->head_dim, d->max_entries + d->window);
}
size_t ws_attention_parts(const csa_dims *d, size_t *off_idx, size_t *off_topk, size_t *off_mqa, bool fp8 = false) {
    const size_t Q = (size_t)n_queries(d);
    const size_t scores = align_up(Q * (size_t)d->max_entries * 4);
    const size_t idx = align_up(Q * (size_t)d->topk * 4);
    *off_idx = scores;
    *off_topk = scores + idx;
    *off_mqa = *off_topk + align_up(ws_topk(d, true, fp8));
    return *off_mqa + align_up(ws_sparse(d)) + 256;
}

csa_status check_ws(void *ws, size_t have, size_t need) {
    if (need == 0) return CSA_OK;
    if (!ws) return fail(CSA_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", need);
    if (have < need) return fail(CSA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
    return CSA_OK;
}

csa_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(CSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

csa::ScoreArgs score_args(const csa_dims *d, const void *q_idx, const float *w, const void *const *k_idx,
                          const int32_t *seq_len, const int32_t *q_pos, float *scores) {
    csa::ScoreArgs a{};
    a.q_idx = q_idx;
    a.w = w;
    a.k_idx = k_idx;
    a.seq_len = seq_len;
    a.q_pos = q_pos;
    a.scores = scores;
    a.B = d->batch;
    a.T = d->q_len;
    a.HI = d->index_heads;
    a.DI = d->index_dim;
    a.ratio = d->ratio;
    a.act = d->index_act;
    a.n_max = d->max_entries;
    return a;
}

csa::TopkArgs topk_args(const csa_dims *d, const float *scores, const int32_t *seq_len, const int32_t *q_pos,
                        int32_t *idx, void *ws, bool fused = false, bool fp8 = false) {
    csa::TopkArgs a{};
    a.scores = scores;
    a.seq_len = seq_len;
    a.q_pos = q_pos;
    a.idx = idx;
    a.B = d->batch;
    a.T = d->q_len;
    a.ratio = d->ratio;
    a.K = d->topk;
    a.n_max = d->max_entries;
    csa::topk_carve(a, ws, n_queries(d), win_count(d, fused, fp8), emit_cap(d, fused, fp8));
    // after the tiled scorer the top-k emits the regions itself, one per entry chunk
    if (a.em_cap > 0 && !fused_decode(d, fp8)) a.em_chunk = csa::tiled_chunk_entries(d->batch, d->q_len, d->max_entries);
    return a;
}

csa::MqaArgs mqa_args(const csa_dims *d, const void *q, const void *const *kv, const void *const *v,
                      const int32_t *topk_idx, const void *const *win, const void *const *win_v,
                      const int32_t *win_pos0, const int32_t *win_rows, const int32_t *seq_len,
                      const int32_t *q_pos, const float *sink, float *out, float *lse, void *ws, int max_rows) {
    csa::MqaArgs a{};
    a.q = q;
    a.kv = kv;
    a.v = v;
    a.topk_idx = topk_idx;
    a.win = win;
    a.win_v = win_v;
    a.win_pos0 = win_pos0;
    a.win_rows = win_rows;
    a.seq_len = seq_len;
    a.q_pos = q_pos;
    a.sink = sink;
    a.out = out;
    a.lse = lse;
    a.B = d->batch;
    a.T = d->q_len;
    a.H = d->n_heads;
    a.D = d->head_dim;
    a.K = d->topk;
    a.W = d->window;
    a.ratio = d->ratio;
    a.scale = scale_of(d);
    a.n_splits = 1;
    a.n_tiles = 1;
    if (d->dtype == CSA_BF16) csa::mqa_plan(n_queries(d), max_rows, &a.n_splits, &a.n_tiles);
    csa::mqa_carve(a, ws, n_queries(d));
    return a;
}

csa_status check_score_ptrs(const void *q_idx, const float *w, const void *const *k_idx, const int32_t *seq_len,
                            const int32_t *q_pos, const float *scores) {
    REQUIRE_PTR(q_idx);
    REQUIRE_PTR(w);
    REQUIRE_PTR(k_idx);
    REQUIRE_PTR(seq_len);
    REQUIRE_PTR(q_pos);
    REQUIRE_PTR(scores);
    REQUIRE_ALIGN(q_idx, 16);
    REQUIRE_ALIGN(w, 16);
    REQUIRE_ALIGN(k_idx, 8);
    REQUIRE_ALIGN(seq_len, 4);
    REQUIRE_ALIGN(q_pos, 4);
    REQUIRE_ALIGN(scores, 16);
    return CSA_OK;
}

csa_status check_attn_ptrs(const void *q, const void *const *kv, const void *const *v, const void *const *win,
                           const void *const *win_v, const int32_t *win_pos0, const int32_t *win_rows,
                           const int32_t *seq_len, const int32_t *q_pos, const float *sink, const float *out,
                           const float *lse) {
    REQUIRE_PTR(q);
    REQUIRE_PTR(kv);
    REQUIRE_PTR(win);
    REQUIRE_PTR(win_pos0);
    REQUIRE_PTR(win_rows);
    REQUIRE_PTR(seq_len);
    REQUIRE_PTR(q_pos);
    REQUIRE_PTR(sink);
    REQUIRE_PTR(out);
    REQUIRE_ALIGN(q, 16);
    REQUIRE_ALIGN(kv, 8);
    REQUIRE_ALIGN(v, 8);
    REQUIRE_ALIGN(win, 8);
    REQUIRE_ALIGN(win_v, 8);
    REQUIRE_ALIGN(win_pos0, 4);
    REQUIRE_ALIGN(win_rows, 4);
    REQUIRE_ALIGN(seq_len, 4);
    REQUIRE_ALIGN(q_pos, 4);
    REQUIRE_ALIGN(sink, 4);
    REQUIRE_ALIGN(out, 16);
    REQUIRE_ALIGN(lse, 4);
    return CSA_OK;
}

}  // namespace

extern "C" {

int32_t csa_abi_version(void) { return CSA_ABI_VERSION; }

const char *csa_last_error(void) { return g_last_error.c_str(); }

const char *csa_status_string(int32_t s) {
    switch (s) {
        case CSA_OK: return "CSA_OK";
        case CSA_ERR_NULL: return "CSA_ERR_NULL: a required pointer is NULL";
        case CSA_ERR_DIM: return "CSA_ERR_DIM: invalid or inconsistent size";
        case CSA_ERR_ALIGN: return "CSA_ERR_ALIGN: misaligned base address";
        case CSA_ERR_UNSUPPORTED: return "CSA_ERR_UNSUPPORTED: dtype/shape combination not implemented";
        case CSA_ERR_WORKSPACE: return "CSA_ERR_WORKSPACE: workspace missing or too small";
        case CSA_ERR_HIP: return "CSA_ERR_HIP: kernel launch failed";
        default: return "unknown csa_status";
    }
}

csa_status csa_workspace_size(const csa_dims *d, int32_t op, size_t *bytes) {
    if (!bytes) return fail(CSA_ERR_NULL, "argument 'bytes' is NULL");
    *bytes = 0;
    csa_status s = check_common(d);
    if (s) return s;
    switch (op) {
        case CSA_OP_INDEX_SCORES:
            if ((s = check_scores(d))) return s;
            *bytes = 0;
            break;
        case CSA_OP_TOPK:
            if ((s = check_topk(d))) return s;
            *bytes = ws_topk(d);
            break;
        case CSA_OP_SPARSE_MQA:
            if ((s = check_topk(d)) || (s = check_attn(d))) return s;
            *bytes = ws_sparse(d);
            break;
        case CSA_OP_HCA_MQA:
            if ((s = check_attn(d))) return s;
            *bytes = ws_hca(d);
            break;
        case CSA_OP_ATTENTION: {
            if ((s = check_scores(d)) || (s = check_topk(d)) || (s = check_attn(d))) return s;
            size_t a, b, c;
            *bytes = ws_attention_parts(d, &a, &b, &c);
            break;
        }
        case CSA_OP_ATTENTION_FP8: {
            if ((s = check_scores_fp8(d)) || (s = check_topk(d)) || (s = check_attn(d))) return s;
            if (d->dtype != CSA_BF16) return fail(CSA_ERR_UNSUPPORTED, "fp8 index path: attention dtype must be bf16");
            size_t a, b, c;
            *bytes = ws_attention_parts(d, &a, &b, &c, true);
            break;
        }
        default: return fail(CSA_ERR_UNSUPPORTED, "unknown op %d", op);
    }
    return ok();
}

csa_status csa_index_scores(const csa_dims *d, const void *q_idx, const float *w, const void *const *k_idx,
                            const int32_t *seq_len, const int32_t *q_pos, float *scores, void *ws, size_t ws_bytes,
                            void *stream) {
    (void)ws;
    (void)ws_bytes;
    csa_status s;
    if ((s = check_common(d)) || (s = check_scores(d))) return s;
    if ((s = check_score_ptrs(q_idx, w, k_idx, seq_len, q_pos, scores))) return s;
    const csa::ScoreArgs a = score_args(d, q_idx, w, k_idx, seq_len, q_pos, scores);
    return hip_status(csa::launch_index_scores(a, d->dtype, (hipStream_t)stream), "csa_index_scores");
}

csa_status csa_index_scores_fp8(const csa_dims *d, const uint8_t *q8, const float *q_scale, const float *w,
                                const void *const *k8, const void *const *k_scale, const int32_t *seq_len,
                                const int32_t *q_pos, float *scores, void *stream) {
    csa_status s;
    if ((s = check_common(d))) return s;
    if ((s = check_scores_fp8(d))) return s;
    if ((s = check_score_ptrs(q8, w, k8, seq_len, q_pos, scores))) return s;
    REQUIRE_PTR(q_scale);
    REQUIRE_PTR(k_scale);
    REQUIRE_ALIGN(q_scale, 4);
    REQUIRE_ALIGN(k_scale, 8);
    csa::ScoreArgs a = score_args(d, q8, w, k8, seq_len, q_pos, scores);
    a.q_scale = q_scale;
    a.k_scale = k_scale;
    return hip_status(csa::launch_index_scores_fp8(a, (hipStream_t)stream), "csa_index_scores_fp8");
}

static csa_status check_compress(const csa_compress_dims *d) {
    if (!d) return fail(CSA_ERR_NULL, "dims is NULL");
    if (d->tokens < 1 || d->n_entries < 1 || d->first_entry < 0 || d->ratio < 1)
        return fail(CSA_ERR_DIM, "tokens, n_entries, ratio must be >= 1 and first_entry >= 0");
    if (d->hidden < 64 || d->hidden % 64) return fail(CSA_ERR_DIM, "hidden must be a positive multiple of 64");
    if (d->out_dim != 128 && d->out_dim != 256 && d->out_dim != 512)
        return fail(CSA_ERR_UNSUPPORTED, "out_dim must be 128, 256 or 512 (got %d)", d->out_dim);
    if (d->window < d->ratio || d->window > 4096) return fail(CSA_ERR_DIM, "window must be in [ratio, 4096]");
    if (d->rope_dims < 0 || d->rope_dims > d->out_dim || (d->rope_dims & 1))
        return fail(CSA_ERR_DIM, "rope_dims must be even and <= out_dim");
    if (d->hadamard != 0 && d->hadamard != 1) return fail(CSA_ERR_DIM, "hadamard must be 0 or 1");
    if (!(d->rope_theta > 0.f) || !(d->rms_eps > 0.f)) return fail(CSA_ERR_DIM, "rope_theta and rms_eps must be > 0");
    if ((long long)d->ratio * ((long long)d->first_entry + d->n_entries) > (1ll << 30))
        return fail(CSA_ERR_DIM, "entry positions beyond 2^30");
    const long long first_tok = (long long)d->ratio * d->first_entry + d->ratio - d->window;
    const long long last_tok = (long long)d->ratio * (d->first_entry + d->n_entries - 1) + d->ratio - 1;
    if ((first_tok < 0 ? 0 : first_tok) < d->pos0 || last_tok >= (long long)d->pos0 + d->tokens)
        return fail(CSA_ERR_DIM, "x rows [%d, %lld) do not cover the window tokens [%lld, %lld]", d->pos0,
                    (long long)d->pos0 + d->tokens, first_tok < 0 ? 0 : first_tok, last_tok);
    return CSA_OK;
}

static size_t ws_compress(const csa_compress_dims *d) {
    const int s = csa::compress_splits(d->tokens, d->hidden, d->out_dim);
    return (size_t)s * d->tokens * 2 * d->out_dim * 4;
}

csa_status csa_compress_workspace_size(const csa_compress_dims *d, size_t *bytes) {
    csa_status s;
    if ((s = check_compress(d))) return s;
    REQUIRE_PTR(bytes);
    *bytes = ws_compress(d);
    return CSA_OK;
}

csa_status csa_compress(const csa_compress_dims *d, const void *x, const void *wkv, const void *wgate,
                        const float *ape, const float *gamma, void *out, void *ws, size_t ws_bytes, void *stream) {
    csa_status s;
    if ((s = check_compress(d))) return s;
    REQUIRE_PTR(x);
    REQUIRE_PTR(wkv);
    REQUIRE_PTR(wgate);
    REQUIRE_PTR(ape);
    REQUIRE_PTR(gamma);
    REQUIRE_PTR(out);
    REQUIRE_ALIGN(x, 16);
    REQUIRE_ALIGN(wkv, 16);
    REQUIRE_ALIGN(wgate, 16);
    REQUIRE_ALIGN(ape, 16);
    REQUIRE_ALIGN(gamma, 16);
    REQUIRE_ALIGN(out, 4);
    if ((s = check_ws(ws, ws_bytes, ws_compress(d)))) return s;
    REQUIRE_ALIGN(ws, 16);
    csa::CompressArgs a{};
    a.x = x;
    a.wkv = wkv;
    a.wgate = wgate;
    a.ape = ape;
    a.gamma = gamma;
    a.out = out;
    a.part = (float *)ws;
    a.tokens = d->tokens;
    a.hidden = d->hidden;
    a.out_dim = d->out_dim;
    a.ratio = d->ratio;
    a.window = d->window;
    a.rope_dims = d->rope_dims;
    a.hadamard = d->hadamard;
    a.first_entry = d->first_entry;
    a.n_entries = d->n_entries;
    a.pos0 = d->pos0;
    a.n_splits = csa::compress_splits(d->tokens, d->hidden, d->out_dim);
    a.rope_theta = d->rope_theta;
    a.rms_eps = d->rms_eps;
    a.rope_ln_theta = std::log((double)d->rope_theta);
    return hip_status(csa::launch_compress(a, (hipStream_t)stream), "csa_compress");
}

csa_status csa_topk_select(const csa_dims *d, const float *scores, const int32_t *seq_len, const int32_t *q_pos,
                           int32_t *topk_idx, void *ws, size_t ws_bytes, void *stream) {
    csa_status s;
    if ((s = check_common(d)) || (s = check_topk(d))) return s;
    REQUIRE_PTR(scores);
    REQUIRE_PTR(seq_len);
    REQUIRE_PTR(q_pos);
    REQUIRE_PTR(topk_idx);
    REQUIRE_ALIGN(scores, 16);
    REQUIRE_ALIGN(seq_len, 4);
    REQUIRE_ALIGN(q_pos, 4);
    REQUIRE_ALIGN(topk_idx, 16);
    if ((s = check_ws(ws, ws_bytes, ws_topk(d)))) return s;
    const csa::TopkArgs a = topk_args(d, scores, seq_len, q_pos, topk_idx, ws);
    return hip_status(csa::launch_topk(a, (hipStream_t)stream), "csa_topk_select");
}

csa_status csa_sparse_mqa_decode(const csa_dims *d, const void *q, const void *const *kv, const void *const *v,
                                 const int32_t *topk_idx, const void *const *win, const void *const *win_v,
                                 const int32_t *win_pos0, const int32_t *win_rows, const int32_t *seq_len,
                                 const int32_t *q_pos, const float *sink, float *out, float *lse, void *ws,
                                 size_t ws_bytes, void *stream) {
    csa_status s;
    if ((s = check_common(d)) || (s = check_topk(d)) || (s = check_attn(d))) return s;
    if ((s = check_attn_ptrs(q, kv, v, win, win_v, win_pos0, win_rows, seq_len, q_pos, sink, out, lse))) return s;
    REQUIRE_PTR(topk_idx);
    REQUIRE_ALIGN(topk_idx, 4);
    if ((s = check_ws(ws, ws_bytes, ws_sparse(d)))) return s;
    const csa::MqaArgs a = mqa_args(d, q, kv, v, topk_idx, win, win_v, win_pos0, win_rows, seq_len, q_pos, sink, out,
                                    lse, ws, d->topk + d->window);
    return hip_status(csa::launch_mqa(a, d->dtype, (hipStream_t)stream), "csa_sparse_mqa_decode");
}

csa_status hca_mqa_decode(const csa_dims *d, const void *q, const void *const *kv, const void *const *v,
                          const void *const *win, const void *const *win_v, const int32_t *win_pos0,
                          const int32_t *win_rows, const int32_t *seq_len, const int32_t *q_pos, const float *sink,
                          float *out, float *lse, void *ws, size_t ws_bytes, void *stream) {
    csa_status s;
    if ((s = check_common(d)) || (s = check_attn(d))) return s;
    if ((s = check_attn_ptrs(q, kv, v, win, win_v, win_pos0, win_rows, seq_len, q_pos, sink, out, lse))) return s;
    if ((s = check_ws(ws, ws_bytes, ws_hca(d)))) return s;
    const csa::MqaArgs a = mqa_args(d, q, kv, v, nullptr, win, win_v, win_pos0, win_rows, seq_len, q_pos, sink, out,
                                    lse, ws, d->max_entries + d->window);
    return hip_status(csa::launch_mqa(a, d->dtype, (hipStream_t)stream), "hca_mqa_decode");
}

csa_status csa_attention(const csa_dims *d, const void *q, const void *q_idx, const float *w,
                         const void *const *k_idx, const void *const *kv, const void *const *v,
                         const void *const *win, const void *const *win_v, const int32_t *win_pos0,
                         const int32_t *win_rows, const int32_t *seq_len, const int32_t *q_pos, const float *sink,
                         float *out, float *lse, int32_t *topk_idx_out, float *scores_out, void *ws,
                         size_t ws_bytes, void *stream) {
    return csa_api::attention_impl(d, q, q_idx, w, k_idx, kv, v, win, win_v, win_pos0, win_rows, seq_len, q_pos,
                                   sink, out, lse, topk_idx_out, scores_out, ws, ws_bytes, stream);
}

csa_status csa_attention_fp8(const csa_dims *d, const void *q, const uint8_t *q8, const float *q_scale,
                             const float *w, const void *const *k8, const void *const *k_scale,
                             const void *const *kv, const void *const *v, const void *const *win,
                             const void *const *win_v, const int32_t *win_pos0, const int32_t *win_rows,
                             const int32_t *seq_len, const int32_t *q_pos, const float *sink, float *out, float *lse,
                             int32_t *topk_idx_out, float *scores_out, void *ws, size_t ws_bytes, void *stream) {
    REQUIRE_PTR(q_scale);
    REQUIRE_PTR(k_scale);
    REQUIRE_ALIGN(q_scale, 4);
    REQUIRE_ALIGN(k_scale, 8);
    const csa_api::IndexFp8 f8{q_scale, k_scale};
    return csa_api::attention_impl(d, q, q8, w, k8, kv, v, win, win_v, win_pos0, win_rows, seq_len, q_pos, sink,
                                   out, lse, topk_idx_out, scores_out, ws, ws_bytes, stream, &f8);
}

}  // extern "C"

csa_status csa_api::attention_impl(const csa_dims *d, const void *q, const void *q_idx, const float *w,
                                   const void *const *k_idx, const void *const *kv, const void *const *v,
                                   const void *const *win, const void *const *win_v, const int32_t *win_pos0,
                                   const int32_t *win_rows, const int32_t *seq_len, const int32_t *q_pos,
                                   const float *sink, float *out, float *lse, int32_t *topk_idx_out,
                                   float *scores_out, void *ws, size_t ws_bytes, void *stream, const IndexFp8 *f8) {
    csa_status s;
    const bool fp8 = f8 != nullptr;
    if ((s = check_common(d)) || (s = fp8 ? check_scores_fp8(d) : check_scores(d)) || (s = check_topk(d)) ||
        (s = check_attn(d)))
        return s;
    if (fp8 && d->dtype != CSA_BF16) return fail(CSA_ERR_UNSUPPORTED, "fp8 index path: attention dtype must be bf16");
    if ((s = check_attn_ptrs(q, kv, v, win, win_v, win_pos0, win_rows, seq_len, q_pos, sink, out, lse))) return s;
    REQUIRE_PTR(q_idx);
    REQUIRE_PTR(w);
    REQUIRE_PTR(k_idx);
    REQUIRE_ALIGN(q_idx, 16);
    REQUIRE_ALIGN(w, 16);
    REQUIRE_ALIGN(k_idx, 8);
    REQUIRE_ALIGN(topk_idx_out, 16);
    REQUIRE_ALIGN(scores_out, 16);
    size_t off_idx, off_topk, off_mqa;
    const size_t need = ws_attention_parts(d, &off_idx, &off_topk, &off_mqa, fp8);
    if ((s = check_ws(ws, ws_bytes, need))) return s;
    REQUIRE_ALIGN(ws, 16);
    char *base = (char *)ws;
    float *scores = scores_out ? scores_out : (float *)base;
    int32_t *idx = topk_idx_out ? topk_idx_out : (int32_t *)(base + off_idx);
    hipStream_t st = (hipStream_t)stream;
    csa::TopkArgs ta = topk_args(d, scores, seq_len, q_pos, idx, base + off_topk, true, fp8);
    csa::ScoreArgs sa = score_args(d, q_idx, w, k_idx, seq_len, q_pos, scores);
    if (fp8) {
        sa.q_scale = f8->q_scale;
        sa.k_scale = f8->k_scale;
    }
    // the scorer also writes the top-k key-histogram windows while it writes the scores
    const bool fused_hist = csa::topk_uses_histogram(d->max_entries) && win_count(d, true, fp8) > 0;
    if (fused_hist) {
        sa.win_hdr = ta.win_hdr;
        sa.win_cnt = ta.win_cnt;
        sa.K = d->topk;
        sa.em_cap = ta.em_cap;  // the decode scorer also hands the selection its high entries
        sa.em_hdr = ta.em_hdr;
        sa.em_key = ta.em_key;
        sa.em_idx = ta.em_idx;
        // many queries per sequence and no score output asked for: the tiled
        // scorer keeps each (query, entry chunk)'s K best entries as it goes
        // and writes no scores; the selection works from those alone
        if (!scores_out && !fused_decode(d, fp8) && ta.em_cap >= d->topk && d->topk <= csa::kSelKeepMax &&
            csa::tiled_chunk_entries(d->batch, d->q_len, d->max_entries) <= csa::kSelChunkMax) {
            sa.sel_stream = 1;
            sa.win_hdr = nullptr;
            sa.win_cnt = nullptr;
            ta.em_stream = 1;
            ta.em_chunk = 0;
        }
    }
    hipError_t e = fp8 ? csa::launch_index_scores_fp8(sa, st) : csa::launch_index_scores(sa, d->dtype, st);
    if (e != hipSuccess) return hip_status(e, "csa_attention/scores");
    e = csa::launch_topk(ta, st, fused_hist);
    if (e != hipSuccess) return hip_status(e, "csa_attention/topk");
    const csa::MqaArgs ma = mqa_args(d, q, kv, v, idx, win, win_v, win_pos0, win_rows, seq_len, q_pos, sink, out, lse,
                                     base + off_mqa, d->topk + d->window);
    return hip_status(csa::launch_mqa(ma, d->dtype, st), "csa_attention/attention");
}
