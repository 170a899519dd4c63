/*
 * CPU oracle for the compressed-sparse-attention (CSA) decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow reference that the HIP
 * path is checked against.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load it; the product library never does.  It shares no
 * code, header, table or helper with the HIP path.
 *
 * Every routine is the plain definition written out with scalar loops and
 * float64 accumulation (bf16 and fp32 inputs convert to float64 exactly).
 * Sources, cited by page title and section:
 *   [A] "DeepSeek-V4 Architecture Analysis" (open-deepseek-v4,
 *       architecture_analysis.py), INNOVATIONS section 1 "Compressed Sparse
 *       Attention": sliding window of the nearest 128 tokens, 4:1 and 128:1
 *       compression, an indexer that scores compressed positions with a
 *       dot product and per-head importance weights and keeps the top-k, and a
 *       learnable per-head scalar sink; section 2 "Unified head dimension":
 *       one 512-d row serves as key and value.
 *   [C] "DeepSeek-V4-Flash-0731" (mic coverage page), config table:
 *       quantization_config (fp8, e4m3 format, dynamic activation scheme).
 *   [D] "DeepSeek-V4-Flash" (llm-atlas), raw config.json table (as [B]):
 *       compress_rope_theta, rms_norm_eps, qk_rope_head_dim.
 *   [B] "DeepSeek-V4-Flash" (llm-atlas), raw config.json table: index_n_heads,
 *       index_head_dim, index_topk, sliding_window, head_dim, 64 q-heads / 1
 *       kv-head.
 * Readings where the pages say nothing (each listed in the design notes):
 *   R1 indexer nonlinearity between the per-head dot product and the weighting
 *      is ReLU (ACT_NONE also offered); no extra scaling constants;
 *   R2 compressed entry j of ratio r covers raw tokens [r*j, r*j+r-1] and is
 *      visible to a query at position p iff r*j+r-1 <= p and j < floor(L/r);
 *   R3 the window is raw positions [max(0,p-W+1), p], including p;
 *   R4 top-k order is (fp32 score desc, index asc); the result is emitted
 *      ascending by index and padded with -1;
 *   R5 one softmax over selected rows then window rows, plus the sink as one
 *      extra logit per head that adds exp(sink) to the denominator only;
 *   R6 softmax scale is a caller value (1/sqrt(D) by default);
 *   R7 fp8 index tensors carry one fp32 scale per row (query-head row, key
 *      entry); the pages name the format but not the scale granularity.
 */
#ifndef CSA_ORACLE_H
#define CSA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };
enum { ORACLE_ACT_RELU = 0, ORACLE_ACT_NONE = 1 };
enum { ORACLE_OK = 0, ORACLE_EINVAL = -1, ORACLE_EWINDOW = -2, ORACLE_ENOMEM = -3 };

/* Threads the oracle's OpenMP loops use. */
int oracle_num_threads(void);

/* Number of compressed entries visible to a query at position pos (R2). */
int64_t oracle_visible_count(int64_t seq_len, int64_t pos, int ratio);

/* Indexer scores (R1, R2), [A] sec. 1 indexer bullet, [B] index_* fields.
 * q_idx [B,T,HI,DI], w [B,T,HI] fp32, k_idx[b] -> [N_b,DI] (host pointers),
 * seq_len [B], q_pos [B*T].  scores [B,T,n_max] fp32: the float64 sum rounded
 * to fp32, -inf where not visible or j >= N_b. */
int oracle_index_scores(int B, int T, int HI, int DI, int ratio, int act, int dtype,
                        const void *q_idx, const float *w, const void *const *k_idx,
                        const int32_t *seq_len, const int32_t *q_pos, int n_max,
                        float *scores);

/* Value of one OCP FP8 E4M3 code (1 sign, 4 exponent bits with bias 7, 3
 * mantissa bits; exponent 0 is subnormal, m * 2^-9; S.1111.111 is NaN; no
 * infinities).  Exact in float64. */
double oracle_e4m3_value(uint8_t code);

/* Indexer scores with fp8 index queries and keys (the next row after the bf16
 * path): [C] quantization_config (fp8, e4m3, dynamic activation scales) and
 * [A] sec. 1 indexer bullet (quantization-aware training).  Reading R7: one
 * fp32 scale per index-query row (query, head) and per key row (entry);
 * value = code value * scale.  q8 [B,T,HI,DI] codes, q_scale [B,T,HI],
 * k8[b] -> [N_b,DI] codes, k_scale[b] -> [N_b].  Then exactly the definition
 * of oracle_index_scores on the dequantized values (float64, rounded once). */
int oracle_index_scores_fp8(int B, int T, int HI, int DI, int ratio, int act, const uint8_t *q8,
                            const float *q_scale, const float *w, const uint8_t *const *k8,
                            const float *const *k_scale, const int32_t *seq_len, const int32_t *q_pos,
                            int n_max, float *scores);

/* Top-k selection (R4), [B] index_topk.  idx [B,T,K]. */
int oracle_topk(int B, int T, int ratio, int K, const float *scores, int n_max,
                const int32_t *seq_len, const int32_t *q_pos, int32_t *idx);

/* Attention of H query heads over an explicit list of n rows (R5).
 * q [H,D]; rows[i] -> [D] key row; vrows[i] -> [D] value row (NULL: V = K);
 * sink [H] (may be NULL: no sink).  out [H,D] float64, lse [H] float64. */
int oracle_attend_rows(int H, int D, int dtype, double scale, const void *q,
                       const void *const *rows, const void *const *vrows, int n,
                       const float *sink, double *out, double *lse);

/* Un-normalised partial of the same attention over a subset of rows, without
 * the sink: m[h] = max z, l[h] = sum exp(z-m), o[h,:] = sum exp(z-m) v. */
int oracle_partial_rows(int H, int D, int dtype, double scale, const void *q,
                        const void *const *rows, const void *const *vrows, int n,
                        double *m, double *l, double *o);

/* Merge S partials [S,H], [S,H], [S,H,D] and the sink into out [H,D], lse [H]. */
int oracle_merge_partials(int S, int H, int D, const double *m, const double *l,
                          const double *o, const float *sink, double *out, double *lse);

/* Sparse MQA over the top-k rows then the window rows (R3, R5), [A] sec. 1-2.
 * q [B,T,H,D]; kv[b], v[b] -> [N_b,D] (v NULL: V = K); win[b], win_v[b] ->
 * [win_rows[b],D], row 0 at raw position win_pos0[b] (win_v NULL: V = K);
 * idx [B,T,K] (-1 = none; every other index must be a visible entry).
 * out [B,T,H,D] float64, lse [B,T,H] float64 (lse may be NULL).
 * Returns ORACLE_EWINDOW when a window position is not in the window buffer. */
int oracle_sparse_mqa(int B, int T, int H, int D, int K, int W, int ratio, int dtype, double scale,
                      const void *q, const void *const *kv, const void *const *v,
                      const void *const *win, const void *const *win_v, const int32_t *win_pos0,
                      const int32_t *win_rows, const int32_t *idx, const int32_t *seq_len,
                      const int32_t *q_pos, const float *sink, double *out, double *lse);

/* HCA: dense MQA over every visible compressed entry (ratio, typically 128)
 * then the window rows, [A] sec. 1 HCA bullet.  Arguments as above. */
int oracle_hca_mqa(int B, int T, int H, int D, int W, int ratio, int dtype, double scale,
                   const void *q, const void *const *kv, const void *const *v,
                   const void *const *win, const void *const *win_v, const int32_t *win_pos0,
                   const int32_t *win_rows, const int32_t *seq_len, const int32_t *q_pos,
                   const float *sink, double *out, double *lse);

/* Whole CSA step: scores -> top-k -> sparse MQA.  scores [B,T,n_max] and
 * idx [B,T,K] are outputs too. */
int oracle_csa_attention(int B, int T, int H, int D, int HI, int DI, int K, int W, int ratio,
                         int act, int dtype, double scale, const void *q, const void *q_idx,
                         const float *w, const void *const *k_idx, const void *const *kv,
                         const void *const *v, const void *const *win, const void *const *win_v,
                         const int32_t *win_pos0, const int32_t *win_rows, const int32_t *seq_len,
                         const int32_t *q_pos, const float *sink, int n_max, float *scores,
                         int32_t *idx, double *out, double *lse);

/* KV / index-key compressor (the step before the path: NEXT-2, NEXT-4), [A]
 * sec. 1: gated pooling of the tokens of a compression window with a learned
 * projection (wkv), gating (wgate), absolute position embeddings within the
 * window (ape), RMSNorm on the output and RoPE on the rope dims; 4:1 with
 * overlapping windows (CSA), 128:1 (HCA); the indexer's own compressor adds a
 * Hadamard rotation.  [D] "DeepSeek-V4-Flash" (llm-atlas) config table:
 * compress_rope_theta 160000, rms_norm_eps 1e-6, qk_rope_head_dim 64.
 * Readings (the pages give the ingredients, not the formula):
 *   R8  entry e of ratio r pools raw tokens [r*e + r - window, r*e + r - 1]
 *       (window = 2r overlapping for CSA, r for HCA); tokens before position
 *       0 do not exist and are left out;
 *   R9  per token t at slot i of the window: kv_t = wkv x_t, gate_t = wgate
 *       x_t + ape[i] (vectors of out_dim); per output dim a softmax over the
 *       window's tokens of gate_t weights the kv_t;
 *   R10 RMSNorm: c / sqrt(mean(c^2) + eps) * gamma;
 *   R11 RoPE on the trailing rope_dims dims: pair (2k, 2k+1) of that slice
 *       rotated by (r*e) * theta^(-2k/rope_dims), position r*e being the
 *       entry's first raw token;
 *   R12 optional normalized Hadamard rotation (Sylvester order out_dim)
 *       applied last.
 * x [tokens, hidden] bf16 with token 0 at raw position pos0; wkv, wgate
 * [out_dim, hidden] bf16; ape [window, out_dim]; gamma [out_dim].  out
 * [n_entries, out_dim] float64 for entries first_entry.. (ORACLE_EWINDOW if a
 * window token is not supplied). */
int oracle_compress(int tokens, int hidden, int out_dim, int ratio, int window, int rope_dims,
                    double rope_theta, double eps, int hadamard, const uint16_t *x, int pos0,
                    const uint16_t *wkv, const uint16_t *wgate, const float *ape, const float *gamma,
                    int first_entry, int n_entries, double *out);

#ifdef __cplusplus
}
#endif
#endif
