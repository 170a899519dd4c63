/*
 * CPU oracle for the CSA decode path -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain scalar loops, float64 accumulation.  Nothing here is blocked, fused or
 * reordered beyond the definitions in oracle.h; OpenMP only spreads
 * independent outputs over threads.  See oracle.h for the sources (cited by
 * page title and section) and the readings R1-R6 taken where they are silent.
 */
#include "oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* One input element as float64 (bf16 and fp32 both convert exactly). */
static double load(const void *p, int dtype, int64_t i) {
    if (dtype == ORACLE_BF16) {
        uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return (double)((const float *)p)[i];
}

static size_t elem_size(int dtype) { return dtype == ORACLE_BF16 ? 2 : 4; }

static const void *row_ptr(const void *base, int dtype, int64_t row, int dim) {
    return (const char *)base + (size_t)row * (size_t)dim * elem_size(dtype);
}

int oracle_num_threads(void) { return omp_get_max_threads(); }

/* R2: entry j covers raw tokens [r*j, r*j+r-1]; only complete spans exist. */
static int entry_visible(int64_t j, int64_t seq_len, int64_t pos, int ratio) {
    return j < seq_len / ratio && (int64_t)ratio * j + ratio - 1 <= pos;
}

int64_t oracle_visible_count(int64_t seq_len, int64_t pos, int ratio) {
    int64_t n = 0;
    for (int64_t j = 0; j < seq_len / ratio; ++j) n += entry_visible(j, seq_len, pos, ratio);
    return n;
}

static int check_query(int64_t seq_len, int64_t pos) { return pos >= 0 && pos < seq_len; }

int oracle_index_scores(int B, int T, int HI, int DI, int ratio, int act, int dtype,
                        const void *q_idx, const float *w, const void *const *k_idx,
                        const int32_t *seq_len, const int32_t *q_pos, int n_max,
                        float *scores) {
    if (B <= 0 || T <= 0 || HI <= 0 || DI <= 0 || ratio <= 0 || n_max <= 0) return ORACLE_EINVAL;
    if (act != ORACLE_ACT_RELU && act != ORACLE_ACT_NONE) return ORACLE_EINVAL;
    if (!q_idx || !w || !k_idx || !seq_len || !q_pos || !scores) return ORACLE_EINVAL;
    for (int bt = 0; bt < B * T; ++bt) {
        int b = bt / T;
        if (!check_query(seq_len[b], q_pos[bt]) || seq_len[b] / ratio > n_max) return ORACLE_EINVAL;
    }
    for (int bt = 0; bt < B * T; ++bt) {
        const int b = bt / T;
        const int64_t L = seq_len[b], p = q_pos[bt];
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < n_max; ++j) {
            if (!entry_visible(j, L, p, ratio)) {
                scores[(int64_t)bt * n_max + j] = -INFINITY;
                continue;
            }
            double s = 0.0;
            for (int h = 0; h < HI; ++h) {
                double dot = 0.0; /* per-head dot product of index query and index key */
                for (int d = 0; d < DI; ++d)
                    dot += load(q_idx, dtype, ((int64_t)bt * HI + h) * DI + d) *
                           load(k_idx[b], dtype, j * DI + d);
                double a = (act == ORACLE_ACT_RELU) ? (dot > 0.0 ? dot : 0.0) : dot;
                s += (double)w[(int64_t)bt * HI + h] * a; /* per-head importance weight */
            }
            scores[(int64_t)bt * n_max + j] = (float)s;
        }
    }
    return ORACLE_OK;
}

typedef struct {
    float s;
    int32_t j;
} scored_t;

/* (score desc, index asc) */
static int by_score_then_index(const void *a, const void *b) {
    const scored_t *x = (const scored_t *)a, *y = (const scored_t *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j > y->j) - (x->j < y->j);
}

static int by_value(const void *a, const void *b) {
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

double oracle_e4m3_value(uint8_t code) {
    const int sign = code >> 7, e = (code >> 3) & 0xF, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);  /* subnormal: m/8 * 2^(1-7) */
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

/* R7: dequantize (code value * row scale, float64), then the score definition. */
int oracle_index_scores_fp8(int B, int T, int HI, int DI, int ratio, int act, const uint8_t *q8,
                            const float *q_scale, const float *w, const uint8_t *const *k8,
                            const float *const *k_scale, const int32_t *seq_len, const int32_t *q_pos,
                            int n_max, float *scores) {
    if (B <= 0 || T <= 0 || HI <= 0 || DI <= 0 || ratio <= 0 || n_max <= 0) return ORACLE_EINVAL;
    if (act != ORACLE_ACT_RELU && act != ORACLE_ACT_NONE) return ORACLE_EINVAL;
    if (!q8 || !q_scale || !w || !k8 || !k_scale || !seq_len || !q_pos || !scores) return ORACLE_EINVAL;
    for (int bt = 0; bt < B * T; ++bt) {
        int b = bt / T;
        if (!check_query(seq_len[b], q_pos[bt]) || seq_len[b] / ratio > n_max) return ORACLE_EINVAL;
    }
    double val[256]; /* code -> value, from the format definition above */
    for (int c = 0; c < 256; ++c) val[c] = oracle_e4m3_value((uint8_t)c);
    for (int bt = 0; bt < B * T; ++bt) {
        const int b = bt / T;
        const int64_t L = seq_len[b], p = q_pos[bt];
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < n_max; ++j) {
            if (!entry_visible(j, L, p, ratio)) {
                scores[(int64_t)bt * n_max + j] = -INFINITY;
                continue;
            }
            const double ks = (double)k_scale[b][j];
            double s = 0.0;
            for (int h = 0; h < HI; ++h) {
                const double qs = (double)q_scale[(int64_t)bt * HI + h];
                double dot = 0.0;
                for (int d = 0; d < DI; ++d)
                    dot += val[q8[((int64_t)bt * HI + h) * DI + d]] * qs * (val[k8[b][j * DI + d]] * ks);
                double a = (act == ORACLE_ACT_RELU) ? (dot > 0.0 ? dot : 0.0) : dot;
                s += (double)w[(int64_t)bt * HI + h] * a;
            }
            scores[(int64_t)bt * n_max + j] = (float)s;
        }
    }
    return ORACLE_OK;
}

int oracle_topk(int B, int T, int ratio, int K, const float *scores, int n_max,
                const int32_t *seq_len, const int32_t *q_pos, int32_t *idx) {
    if (B <= 0 || T <= 0 || ratio <= 0 || K <= 0 || n_max <= 0) return ORACLE_EINVAL;
    if (!scores || !seq_len || !q_pos || !idx) return ORACLE_EINVAL;
    for (int bt = 0; bt < B * T; ++bt) {
        int b = bt / T;
        if (!check_query(seq_len[b], q_pos[bt]) || seq_len[b] / ratio > n_max) return ORACLE_EINVAL;
    }
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bt = 0; bt < B * T; ++bt) {
        const int b = bt / T;
        scored_t *c = (scored_t *)malloc(sizeof(scored_t) * (size_t)n_max);
        int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
        if (!c || !sel) {
            free(c);
            free(sel);
#pragma omp atomic write
            err = 1;
            continue;
        }
        int m = 0;
        for (int j = 0; j < n_max; ++j)
            if (entry_visible(j, seq_len[b], q_pos[bt], ratio)) {
                c[m].s = scores[(int64_t)bt * n_max + j];
                c[m].j = j;
                ++m;
            }
        qsort(c, (size_t)m, sizeof(scored_t), by_score_then_index);
        int k = m < K ? m : K;
        for (int i = 0; i < k; ++i) sel[i] = c[i].j;
        qsort(sel, (size_t)k, sizeof(int32_t), by_value);
        for (int i = 0; i < K; ++i) idx[(int64_t)bt * K + i] = i < k ? sel[i] : -1;
        free(c);
        free(sel);
    }
    return err ? ORACLE_ENOMEM : ORACLE_OK;
}

int oracle_attend_rows(int H, int D, int dtype, double scale, const void *q,
                       const void *const *rows, const void *const *vrows, int n,
                       const float *sink, double *out, double *lse) {
    if (H <= 0 || D <= 0 || n < 0 || !q || (n > 0 && !rows) || !out) return ORACLE_EINVAL;
    int err = 0;
#pragma omp parallel for schedule(static)
    for (int h = 0; h < H; ++h) {
        double *z = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        if (!z) {
#pragma omp atomic write
            err = 1;
            continue;
        }
        const double sk = sink ? (double)sink[h] : -INFINITY;
        double m = sk;
        for (int i = 0; i < n; ++i) {
            double dot = 0.0;
            for (int d = 0; d < D; ++d)
                dot += load(q, dtype, (int64_t)h * D + d) * load(rows[i], dtype, d);
            z[i] = scale * dot;
            if (z[i] > m) m = z[i];
        }
        /* softmax denominator: every row plus the sink logit (no value vector) */
        double l = exp(sk - m);
        for (int i = 0; i < n; ++i) l += exp(z[i] - m);
        for (int d = 0; d < D; ++d) {
            double acc = 0.0;
            for (int i = 0; i < n; ++i)
                acc += exp(z[i] - m) * load(vrows ? vrows[i] : rows[i], dtype, d);
            out[(int64_t)h * D + d] = acc / l;
        }
        if (lse) lse[h] = m + log(l);
        free(z);
    }
    return err ? ORACLE_ENOMEM : ORACLE_OK;
}

int oracle_partial_rows(int H, int D, int dtype, double scale, const void *q,
                        const void *const *rows, const void *const *vrows, int n,
                        double *m, double *l, double *o) {
    if (H <= 0 || D <= 0 || n < 0 || !q || (n > 0 && !rows) || !m || !l || !o) return ORACLE_EINVAL;
    for (int h = 0; h < H; ++h) {
        double *z = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        if (!z) return ORACLE_ENOMEM;
        double mh = -INFINITY;
        for (int i = 0; i < n; ++i) {
            double dot = 0.0;
            for (int d = 0; d < D; ++d)
                dot += load(q, dtype, (int64_t)h * D + d) * load(rows[i], dtype, d);
            z[i] = scale * dot;
            if (z[i] > mh) mh = z[i];
        }
        double lh = 0.0;
        for (int i = 0; i < n; ++i) lh += exp(z[i] - mh);
        for (int d = 0; d < D; ++d) {
            double acc = 0.0;
            for (int i = 0; i < n; ++i)
                acc += exp(z[i] - mh) * load(vrows ? vrows[i] : rows[i], dtype, d);
            o[(int64_t)h * D + d] = acc;
        }
        m[h] = mh;
        l[h] = lh;
        free(z);
    }
    return ORACLE_OK;
}

int oracle_merge_partials(int S, int H, int D, const double *m, const double *l,
                          const double *o, const float *sink, double *out, double *lse) {
    if (S < 0 || H <= 0 || D <= 0 || (S > 0 && (!m || !l || !o)) || !out) return ORACLE_EINVAL;
    for (int h = 0; h < H; ++h) {
        const double sk = sink ? (double)sink[h] : -INFINITY;
        double M = sk;
        for (int s = 0; s < S; ++s)
            if (l[(int64_t)s * H + h] > 0.0 && m[(int64_t)s * H + h] > M) M = m[(int64_t)s * H + h];
        double L = exp(sk - M); /* the sink is counted once, not once per part */
        for (int s = 0; s < S; ++s)
            if (l[(int64_t)s * H + h] > 0.0) L += l[(int64_t)s * H + h] * exp(m[(int64_t)s * H + h] - M);
        for (int d = 0; d < D; ++d) {
            double acc = 0.0;
            for (int s = 0; s < S; ++s)
                if (l[(int64_t)s * H + h] > 0.0)
                    acc += o[((int64_t)s * H + h) * D + d] * exp(m[(int64_t)s * H + h] - M);
            out[(int64_t)h * D + d] = acc / L;
        }
        if (lse) lse[h] = M + log(L);
    }
    return ORACLE_OK;
}

/* Append the window rows of a query at position pos (R3). */
static int add_window(int W, int dtype, int D, int64_t pos, const void *win, const void *win_v,
                      int64_t pos0, int64_t n_rows, const void **rows, const void **vrows, int *n) {
    int64_t lo = pos - W + 1 > 0 ? pos - W + 1 : 0;
    for (int64_t t = lo; t <= pos; ++t) {
        if (t < pos0 || t >= pos0 + n_rows) return ORACLE_EWINDOW;
        rows[*n] = row_ptr(win, dtype, t - pos0, D);
        vrows[*n] = row_ptr(win_v ? win_v : win, dtype, t - pos0, D);
        ++*n;
    }
    return ORACLE_OK;
}

int oracle_sparse_mqa(int B, int T, int H, int D, int K, int W, int ratio, int dtype, double scale,
                      const void *q, const void *const *kv, const void *const *v,
                      const void *const *win, const void *const *win_v, const int32_t *win_pos0,
                      const int32_t *win_rows, const int32_t *idx, const int32_t *seq_len,
                      const int32_t *q_pos, const float *sink, double *out, double *lse) {
    if (B <= 0 || T <= 0 || H <= 0 || D <= 0 || K <= 0 || W <= 0 || ratio <= 0) return ORACLE_EINVAL;
    if (!q || !kv || !win || !win_pos0 || !win_rows || !idx || !seq_len || !q_pos || !out)
        return ORACLE_EINVAL;
    const void **rows = (const void **)malloc(sizeof(void *) * (size_t)(K + W));
    const void **vrows = (const void **)malloc(sizeof(void *) * (size_t)(K + W));
    if (!rows || !vrows) {
        free(rows);
        free(vrows);
        return ORACLE_ENOMEM;
    }
    int rc = ORACLE_OK;
    for (int bt = 0; bt < B * T && rc == ORACLE_OK; ++bt) {
        const int b = bt / T;
        const int64_t L = seq_len[b], p = q_pos[bt];
        if (!check_query(L, p)) { rc = ORACLE_EINVAL; break; }
        int n = 0;
        for (int k = 0; k < K; ++k) { /* selected compressed rows, as given (ascending) */
            int32_t j = idx[(int64_t)bt * K + k];
            if (j < 0) continue;
            if (!entry_visible(j, L, p, ratio)) { rc = ORACLE_EINVAL; break; }
            rows[n] = row_ptr(kv[b], dtype, j, D);
            vrows[n] = row_ptr(v ? v[b] : kv[b], dtype, j, D);
            ++n;
        }
        if (rc != ORACLE_OK) break;
        rc = add_window(W, dtype, D, p, win[b], win_v ? win_v[b] : NULL, win_pos0[b], win_rows[b],
                        rows, vrows, &n);
        if (rc != ORACLE_OK) break;
        rc = oracle_attend_rows(H, D, dtype, scale, row_ptr(q, dtype, (int64_t)bt * H, D), rows, vrows,
                                n, sink, out + (int64_t)bt * H * D, lse ? lse + (int64_t)bt * H : NULL);
    }
    free(rows);
    free(vrows);
    return rc;
}

int oracle_hca_mqa(int B, int T, int H, int D, int W, int ratio, int dtype, double scale,
                   const void *q, const void *const *kv, const void *const *v,
                   const void *const *win, const void *const *win_v, const int32_t *win_pos0,
                   const int32_t *win_rows, const int32_t *seq_len, const int32_t *q_pos,
                   const float *sink, double *out, double *lse) {
    if (B <= 0 || T <= 0 || H <= 0 || D <= 0 || W <= 0 || ratio <= 0) return ORACLE_EINVAL;
    if (!q || !kv || !win || !win_pos0 || !win_rows || !seq_len || !q_pos || !out) return ORACLE_EINVAL;
    int rc = ORACLE_OK;
    for (int bt = 0; bt < B * T && rc == ORACLE_OK; ++bt) {
        const int b = bt / T;
        const int64_t L = seq_len[b], p = q_pos[bt];
        if (!check_query(L, p)) return ORACLE_EINVAL;
        const int64_t cap = L / ratio + W;
        const void **rows = (const void **)malloc(sizeof(void *) * (size_t)cap);
        const void **vrows = (const void **)malloc(sizeof(void *) * (size_t)cap);
        if (!rows || !vrows) {
            free(rows);
            free(vrows);
            return ORACLE_ENOMEM;
        }
        int n = 0;
        for (int64_t j = 0; j < L / ratio; ++j) /* every visible compressed entry, ascending */
            if (entry_visible(j, L, p, ratio)) {
                rows[n] = row_ptr(kv[b], dtype, j, D);
                vrows[n] = row_ptr(v ? v[b] : kv[b], dtype, j, D);
                ++n;
            }
        rc = add_window(W, dtype, D, p, win[b], win_v ? win_v[b] : NULL, win_pos0[b], win_rows[b],
                        rows, vrows, &n);
        if (rc == ORACLE_OK)
            rc = oracle_attend_rows(H, D, dtype, scale, row_ptr(q, dtype, (int64_t)bt * H, D), rows,
                                    vrows, n, sink, out + (int64_t)bt * H * D,
                                    lse ? lse + (int64_t)bt * H : NULL);
        free(rows);
        free(vrows);
    }
    return rc;
}

int oracle_csa_attention(int B, int T, int H, int D, int HI, int DI, int K, int W, int ratio,
                         int act, int dtype, double scale, const void *q, const void *q_idx,
                         const float *w, const void *const *k_idx, const void *const *kv,
                         const void *const *v, const void *const *win, const void *const *win_v,
                         const int32_t *win_pos0, const int32_t *win_rows, const int32_t *seq_len,
                         const int32_t *q_pos, const float *sink, int n_max, float *scores,
                         int32_t *idx, double *out, double *lse) {
    int rc = oracle_index_scores(B, T, HI, DI, ratio, act, dtype, q_idx, w, k_idx, seq_len, q_pos,
                                 n_max, scores);
    if (rc != ORACLE_OK) return rc;
    rc = oracle_topk(B, T, ratio, K, scores, n_max, seq_len, q_pos, idx);
    if (rc != ORACLE_OK) return rc;
    return oracle_sparse_mqa(B, T, H, D, K, W, ratio, dtype, scale, q, kv, v, win, win_v, win_pos0,
                             win_rows, idx, seq_len, q_pos, sink, out, lse);
}
