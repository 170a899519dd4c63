/*
 * libcsa -- compressed sparse attention (CSA) decode path for AMD MI355X (gfx950).
 *
 * C ABI.  Every pointer argument is a plain pointer; "device" means HIP device
 * memory, "host" means ordinary host memory.  No torch or HIP type appears in a
 * signature: the stream is a hipStream_t passed as void* (NULL = null stream).
 *
 * What the path computes (sources cited by page title and section):
 *   [A] "DeepSeek-V4 Architecture Analysis" (open-deepseek-v4
 *       architecture_analysis.py), INNOVATIONS 1 "Compressed Sparse Attention":
 *       a sliding window over the nearest 128 raw tokens; 4:1 compressed KV
 *       entries; 128:1 heavily compressed entries (HCA); an indexer that scores
 *       compressed positions with a dot product and per-head importance
 *       weights and keeps the top-k; a learnable per-head scalar sink.
 *       INNOVATIONS 2 "Unified head dimension": one 512-d row is both key and
 *       value.
 *   [B] "DeepSeek-V4-Flash" (llm-atlas), raw config.json table: head_dim 512,
 *       64 query heads / 1 KV head, index_n_heads 64, index_head_dim 128,
 *       index_topk 512, sliding_window 128.
 *   [C] "DeepSeek-V4-Flash-0731" (mic coverage page), config table:
 *       quantization_config (fp8, E4M3 format, dynamic activation scheme).
 * Readings where the pages are silent:
 *   - indexer activation between the per-head dot product and the weighting:
 *     ReLU (CSA_ACT_RELU, default) or none (CSA_ACT_NONE); no other constants;
 *   - compressed entry j of ratio r covers raw tokens [r*j, r*j+r-1]; a query
 *     at raw position p sees it iff r*j+r-1 <= p and j < floor(L/r);
 *   - the window is raw positions [max(0, p-W+1), p] (the query's own token
 *     included);
 *   - top-k orders by (fp32 score desc, index asc); output is ascending by
 *     index with -1 padding when fewer than K entries are visible;
 *   - one softmax over the selected rows, then the window rows, plus the sink
 *     as one extra logit per head that adds exp(sink) to the denominator only
 *     (no value vector), counted once per (query, head);
 *   - softmax scale defaults to 1/sqrt(head_dim); the sink is not scaled.
 *
 * Ownership and execution: the caller owns every buffer, including the device
 * arrays of per-sequence pointers and the workspace.  The library never
 * allocates device memory, never synchronizes, and keeps no pointer after a
 * call returns.  Work is enqueued on `stream`; buffers must stay alive until
 * the stream passes the call.  Calls are thread-safe (no shared state except
 * a thread-local error string); the one exception is csa_attention_noalloc,
 * whose work area is a static device array of the library shared by every
 * call on a GPU (see there).
 *
 * Errors: all argument checks run on the host before anything is enqueued; on
 * error nothing is launched and the status says why (details in
 * csa_last_error()).  A failed launch returns CSA_ERR_HIP.  Device-side faults
 * surface at the caller's next synchronization.  Per-sequence values held in
 * device memory (seq_len, q_pos, window spans, top-k indices) cannot be checked
 * on the host: kernels clamp every access to the buffer they were given
 * (entries j >= floor(L/r), indices out of range and window positions outside
 * the window buffer are skipped), so such caller mistakes give wrong results,
 * never out-of-bounds accesses, provided the per-sequence buffers really hold
 * floor(L_b/r) rows (caches) and win_rows[b] rows (windows).
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 1

typedef enum csa_status {
    CSA_OK = 0,
    CSA_ERR_NULL = 1,        /* a required pointer is NULL */
    CSA_ERR_DIM = 2,         /* a size is <= 0, inconsistent or too large */
    CSA_ERR_ALIGN = 3,       /* a base address is not 16-byte aligned */
    CSA_ERR_UNSUPPORTED = 4, /* valid but not implemented (dtype/dims combination) */
    CSA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than csa_workspace_size() */
    CSA_ERR_HIP = 6          /* a kernel launch failed */
} csa_status;

typedef enum csa_dtype {
    CSA_F32 = 0,  /* float32 activations and caches (small shapes, VALU kernels) */
    CSA_BF16 = 1  /* bfloat16 activations and caches (MFMA kernels) */
} csa_dtype;

typedef enum csa_index_act { CSA_ACT_RELU = 0, CSA_ACT_NONE = 1 } csa_index_act;

typedef enum csa_op {
    CSA_OP_INDEX_SCORES = 0,
    CSA_OP_TOPK = 1,
    CSA_OP_SPARSE_MQA = 2,
    CSA_OP_HCA_MQA = 3,
    CSA_OP_ATTENTION = 4,
    CSA_OP_ATTENTION_FP8 = 5  /* csa_attention_fp8 */
} csa_op;

/* Problem sizes (host struct). */
typedef struct csa_dims {
    int32_t batch;         /* B sequences */
    int32_t q_len;         /* T query tokens per sequence (1 = decode) */
    int32_t n_heads;       /* H query heads sharing one KV head */
    int32_t head_dim;      /* D, key = value width */
    int32_t index_heads;   /* HI indexer heads */
    int32_t index_dim;     /* DI indexer width */
    int32_t topk;          /* K entries kept per query */
    int32_t window;        /* W raw tokens of the sliding window */
    int32_t ratio;         /* r raw tokens per compressed entry (4 CSA, 128 HCA) */
    int32_t max_entries;   /* host-side bound >= max_b floor(L_b/r): score row stride, grid size */
    int32_t dtype;         /* csa_dtype of q, q_idx, k_idx, kv, v, win, win_v */
    int32_t index_act;     /* csa_index_act */
    float softmax_scale;   /* 0 => 1/sqrt(head_dim) */
} csa_dims;

/*
 * Supported shapes.
 *   CSA_BF16: head_dim 512, index_dim 128, index_heads 64, n_heads 64 (Flash)
 *             or 128 (Pro: [A] ARCHITECTURE_SPEC, DeepSeek-V4-Pro num_heads).
 *   CSA_F32:  head_dim <= 512, index_dim <= 128, index_heads <= 64,
 *             n_heads <= 128 (plain VALU kernels for small fixtures).
 * Limits for both: 1 <= topk <= 2048, window >= 1, ratio >= 1,
 * batch * q_len <= 2^20, max_entries <= 2^26.
 */

/* Device workspace bytes that `op` needs for `dims` (host-only, no HIP call). */
csa_status csa_workspace_size(const csa_dims *dims, int32_t op, size_t *bytes);

/*
 * Indexer scores -- [A] INNOVATIONS 1, indexer bullet; [B] index_* fields.
 *   s[b,t,j] = sum_h w[b,t,h] * act( sum_d q_idx[b,t,h,d] * k_idx_b[j,d] )
 * for visible j, -inf otherwise (including floor(L_b/r) <= j < max_entries).
 *   q_idx   device [B,T,HI,DI] dtype
 *   w       device [B,T,HI] float32 importance weights
 *   k_idx   device array of B device pointers, k_idx[b] -> [floor(L_b/r), DI] dtype
 *   seq_len device [B] int32 raw lengths L_b
 *   q_pos   device [B*T] int32 raw positions p (0 <= p < L_b)
 *   scores  device [B,T,max_entries] float32 (output)
 * Accumulation is fp32 (bf16 products are exact in fp32).
 */
csa_status csa_index_scores(const csa_dims *dims, const void *q_idx, const float *w,
                            const void *const *k_idx, const int32_t *seq_len,
                            const int32_t *q_pos, float *scores, void *workspace,
                            size_t ws_bytes, void *stream);

/*
 * Indexer scores with fp8 index tensors -- the same definition as
 * csa_index_scores on dequantized values; [C] "DeepSeek-V4-Flash-0731"
 * config table, quantization_config (fp8, E4M3 format, dynamic activation
 * scales), and [A] INNOVATIONS 1, indexer bullet (quantization-aware
 * training).  Reading: one fp32 scale per index-query row (query, head) and
 * per key row (entry); a value is code * scale.
 *   q8      device [B,T,HI,DI] uint8 OCP FP8 E4M3 codes (16-byte aligned)
 *   q_scale device [B,T,HI] float32, > 0
 *   w       device [B,T,HI] float32 importance weights
 *   k8      device array of B device pointers, k8[b] -> [floor(L_b/r), DI] codes
 *   k_scale device array of B device pointers, k_scale[b] -> [floor(L_b/r)] float32, > 0
 *   seq_len, q_pos, scores: as csa_index_scores.
 * Requires index_heads 64 and index_dim 128 (dims->dtype is not used).
 * Scales must be positive (ReLU then commutes with them); NaN codes are not
 * checked.  fp8 x fp8 products are exact in fp32; accumulation is fp32.
 */
csa_status csa_index_scores_fp8(const csa_dims *dims, const uint8_t *q8, const float *q_scale,
                                const float *w, const void *const *k8, const void *const *k_scale,
                                const int32_t *seq_len, const int32_t *q_pos, float *scores,
                                void *stream);

/*
 * Top-k selection -- [B] index_topk; [A] INNOVATIONS 1, indexer bullet.
 * Per query: the K visible entries with the largest fp32 score, ties to the
 * lower index; written ascending by index, -1 padding when fewer are visible.
 * Exact: equal to sorting by (score desc, index asc).  -0.0 counts as +0.0;
 * NaN scores are not supported.
 *   scores   device [B,T,max_entries] float32
 *   topk_idx device [B,T,K] int32 (output)
 */
csa_status csa_topk_select(const csa_dims *dims, const float *scores, const int32_t *seq_len,
                           const int32_t *q_pos, int32_t *topk_idx, void *workspace,
                           size_t ws_bytes, void *stream);

/*
 * Sparse multi-query attention with sink -- [A] INNOVATIONS 1 (window,
 * selected compressed rows, sink) and 2 (K = V); [B] 64 q-heads / 1 kv-head.
 * Rows, in order: kv_b[topk_idx[b,t,k]] for k = 0..K-1 (-1 skipped), then the
 * window rows of positions max(0,p-W+1)..p.  One softmax with the sink.
 *   q        device [B,T,H,D] dtype
 *   kv       device array of B device pointers -> [floor(L_b/r), D] (keys; values when v == NULL)
 *   v        NULL, or device array of B device pointers -> [floor(L_b/r), D] values
 *   topk_idx device [B,T,K] int32
 *   win      device array of B device pointers -> [win_rows[b], D], row i = raw position win_pos0[b]+i
 *   win_v    NULL, or as win (window values)
 *   win_pos0, win_rows  device [B] int32
 *   seq_len, q_pos      device [B], [B*T] int32
 *   sink     device [H] float32 logits
 *   out      device [B,T,H,D] float32 (output)
 *   lse      NULL, or device [B,T,H] float32 natural-log sum of exp incl. the sink (output)
 * bf16 path: QK in bf16 MFMA, softmax in fp32, PV in bf16 MFMA on V as given
 * with the weights split into a bf16 high part and a bf16 remainder (about 16
 * significant bits), fp32 accumulation.  Split partials O/l are kept in fp16,
 * each head's values of a 256-dim half scaled by a power of two into
 * [2^14, 2^15) (the inverse kept in fp32), combined in fp32; fp32 output.
 */
csa_status csa_sparse_mqa_decode(const csa_dims *dims, const void *q, const void *const *kv,
                                 const void *const *v, const int32_t *topk_idx,
                                 const void *const *win, const void *const *win_v,
                                 const int32_t *win_pos0, const int32_t *win_rows,
                                 const int32_t *seq_len, const int32_t *q_pos, const float *sink,
                                 float *out, float *lse, void *workspace, size_t ws_bytes,
                                 void *stream);

/*
 * HCA dense multi-query attention with sink -- [A] INNOVATIONS 1, HCA bullet.
 * As csa_sparse_mqa_decode, with rows = every visible entry of the ratio-r
 * cache (r = dims->ratio, typically 128) in ascending order, then the window.
 */
csa_status hca_mqa_decode(const csa_dims *dims, const void *q, const void *const *kv,
                          const void *const *v, const void *const *win, const void *const *win_v,
                          const int32_t *win_pos0, const int32_t *win_rows, const int32_t *seq_len,
                          const int32_t *q_pos, const float *sink, float *out, float *lse,
                          void *workspace, size_t ws_bytes, void *stream);

/*
 * Whole CSA step: csa_index_scores -> csa_topk_select -> csa_sparse_mqa_decode,
 * enqueued on one stream.  topk_idx_out (device [B,T,K] int32) and scores_out
 * (device [B,T,max_entries] float32) are optional outputs; when NULL the
 * intermediates live in the workspace.  With bf16 index tensors the scorer
 * also writes the selection's key-histogram windows (one launch fewer); the
 * selected indices equal csa_topk_select's on the same scores.  With many
 * queries per sequence (q_len >= 8), K <= 512 and scores_out NULL, the scorer
 * writes no scores at all when the chunk plan allows it (entry chunks x K <=
 * 8192, at most 65,536 entries per chunk): each (query, entry chunk) keeps its
 * K best entries as it goes and the selection works from those, with the same
 * result; the workspace's score area is then left untouched.
 */
csa_status csa_attention(const csa_dims *dims, const void *q, const void *q_idx, const float *w,
                         const void *const *k_idx, const void *const *kv, const void *const *v,
                         const void *const *win, const void *const *win_v,
                         const int32_t *win_pos0, const int32_t *win_rows,
                         const int32_t *seq_len, const int32_t *q_pos, const float *sink,
                         float *out, float *lse, int32_t *topk_idx_out, float *scores_out,
                         void *workspace, size_t ws_bytes, void *stream);

/*
 * Whole CSA step with fp8 index tensors: csa_index_scores_fp8 ->
 * csa_topk_select -> csa_sparse_mqa_decode on one stream, the fp8 form of
 * csa_attention ([C] quantization_config: fp8 E4M3; [A] INNOVATIONS 1, the
 * indexer in low precision).  The index query and keys are E4M3 codes with
 * per-row scales, as csa_index_scores_fp8 (q8 16-byte aligned, every k8[b]
 * 16-byte aligned); the attention side (q, kv, v, win, win_v) is bf16, so
 * dims->dtype must be CSA_BF16, with index_heads 64 and index_dim 128.  The
 * fp8 scorer writes the selection's histogram windows and emitted entries as
 * the bf16 decode scorer does, for every query count (no GEMM-tiled fp8
 * scorer: many queries per sequence work but re-read the keys per query).
 * Workspace: csa_workspace_size with CSA_OP_ATTENTION_FP8.  Other arguments,
 * outputs and errors as csa_attention.
 */
csa_status csa_attention_fp8(const csa_dims *dims, const void *q, const uint8_t *q8, const float *q_scale,
                             const float *w, const void *const *k8, const void *const *k_scale,
                             const void *const *kv, const void *const *v, const void *const *win,
                             const void *const *win_v, const int32_t *win_pos0, const int32_t *win_rows,
                             const int32_t *seq_len, const int32_t *q_pos, const float *sink, float *out,
                             float *lse, int32_t *topk_idx_out, float *scores_out, void *workspace,
                             size_t ws_bytes, void *stream);

/*
 * csa_attention without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture that may not allocate, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments, results and
 * errors as csa_attention, minus (workspace, ws_bytes): the work area is a
 * device array of 64 MiB inside the library, one per GPU it runs on, held until
 * the process ends.  Sizes whose work area (csa_workspace_size with
 * CSA_OP_ATTENTION) exceeds 64 MiB return CSA_ERR_WORKSPACE before anything is
 * enqueued; the decode shapes fit (batch 4 at 262,144 entries needs about
 * 7 MiB), a 2,048-query prefill chunk over 262,144 entries does not.  The call
 * allocates nothing; the first call on a device looks up the array's address
 * there.  `stream` must belong to the current device (else
 * CSA_ERR_UNSUPPORTED).  Every call on a GPU shares that GPU's array: calls
 * that overlap on one GPU (other streams or threads) race and must be
 * serialized by the caller.
 */
csa_status csa_attention_noalloc(const csa_dims *dims, const void *q, const void *q_idx, const float *w,
                                 const void *const *k_idx, const void *const *kv, const void *const *v,
                                 const void *const *win, const void *const *win_v,
                                 const int32_t *win_pos0, const int32_t *win_rows,
                                 const int32_t *seq_len, const int32_t *q_pos, const float *sink,
                                 float *out, float *lse, int32_t *topk_idx_out, float *scores_out,
                                 void *stream);

/*
 * KV / index-key compressor -- the step that produces the compressed caches
 * the path reads ([A] INNOVATIONS 1, CSA and HCA bullets: learned projection
 * wkv and gating wgate, absolute position embeddings within each compression
 * window, RMSNorm on the compressed output, RoPE on the rope dims, 4:1 with
 * overlapping windows and 128:1; the indexer's own compressor adds a
 * Hadamard rotation; [B] compress_rope_theta 160000, rms_norm_eps 1e-6).
 * Readings (the pages list the ingredients, not the formula):
 *   - entry e pools raw tokens [r*e + r - window, r*e + r - 1] (window = 2r
 *     overlapping for CSA, r for HCA), tokens before position 0 left out;
 *   - per token t at window slot i: kv_t = wkv x_t, gate_t = wgate x_t +
 *     ape[i]; per output dim a softmax over the window's tokens of gate_t
 *     weights kv_t;
 *   - RMSNorm c / sqrt(mean(c^2) + eps) * gamma;
 *   - RoPE on the trailing rope_dims dims, pair (2k, 2k+1) rotated by
 *     (r*e) * theta^(-2k/rope_dims);
 *   - optional normalized Hadamard rotation (Sylvester order), last.
 */
typedef struct csa_compress_dims {
    int32_t tokens;       /* rows of x: raw positions pos0 .. pos0 + tokens - 1 */
    int32_t hidden;       /* hidden size, a multiple of 64 */
    int32_t out_dim;      /* 128, 256 or 512 */
    int32_t ratio;        /* r >= 1 */
    int32_t window;       /* tokens pooled per entry, ratio <= window <= 4096 */
    int32_t rope_dims;    /* even, <= out_dim (0: no RoPE) */
    int32_t hadamard;     /* 0 or 1 */
    int32_t first_entry;  /* first entry to produce (>= 0) */
    int32_t n_entries;    /* entries to produce (>= 1) */
    int32_t pos0;         /* raw position of x's row 0 */
    float rope_theta;     /* > 0 */
    float rms_eps;        /* > 0 */
} csa_compress_dims;

/* Workspace bytes of csa_compress (host-only). */
csa_status csa_compress_workspace_size(const csa_compress_dims *dims, size_t *bytes);

/*
 *   x      device [tokens, hidden] bf16 (16-byte aligned); every window token
 *          of every requested entry (at raw position >= 0) must be a row of x
 *   wkv, wgate device [out_dim, hidden] bf16 (16-byte aligned)
 *   ape    device [window, out_dim] float32; gamma device [out_dim] float32
 *          (both 16-byte aligned)
 *   out    device [n_entries, out_dim] bf16 (entries first_entry ..)
 *   workspace device, csa_compress_workspace_size bytes (16-byte aligned): the
 *          fp32 projections of x's rows
 * All buffers stay owned by the caller; nothing is allocated.  Shape, pointer,
 * alignment and workspace errors return before anything is enqueued.
 * Projections accumulate in fp32; softmax, norm and rotations in fp32 (RoPE
 * angles in fp64); the result is rounded to bf16.
 */
csa_status csa_compress(const csa_compress_dims *dims, const void *x, const void *wkv, const void *wgate,
                        const float *ape, const float *gamma, void *out, void *workspace, size_t ws_bytes,
                        void *stream);

/* Static string for a status code. */
const char *csa_status_string(int32_t status);

/* Detail of the last error on the calling thread ("" if none). */
const char *csa_last_error(void);

/* CSA_ABI_VERSION of the loaded library. */
int32_t csa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif
