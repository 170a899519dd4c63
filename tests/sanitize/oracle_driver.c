/* Exercises every entry point of the CPU oracle on small inputs, including
 * the degenerate cases (a sequence with no compressed entry, top-k larger
 * than what is visible, an empty row list, several causal queries per
 * sequence) and its argument checks.  Built with AddressSanitizer and
 * UndefinedBehaviorSanitizer by the test suite: every buffer is its own heap
 * allocation of exactly the documented size, so a read or write past one is
 * reported.  Prints "ok" and exits 0 when every call returned what it should. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t g_state = 0x9e3779b97f4a7c15ull;

static double uniform(void) { /* xorshift64*, in [0, 1) */
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (double)((g_state * 0x2545f4914f6cdd1dull) >> 11) * (1.0 / 9007199254740992.0);
}

static uint16_t to_bf16(float f) { /* truncation: any bf16 value will do here */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static void *xalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

/* n values of the given dtype, uniform in [-1, 1) */
static void *values(size_t n, int dtype) {
    if (dtype == ORACLE_F32) {
        float *p = xalloc(n * sizeof(float));
        for (size_t i = 0; i < n; ++i) p[i] = (float)(2.0 * uniform() - 1.0);
        return p;
    }
    uint16_t *p = xalloc(n * sizeof(uint16_t));
    for (size_t i = 0; i < n; ++i) p[i] = to_bf16((float)(2.0 * uniform() - 1.0));
    return p;
}

static float *floats(size_t n, float lo, float hi) {
    float *p = xalloc(n * sizeof(float));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * (float)uniform();
    return p;
}

static int g_failures = 0;

static void expect(int got, int want, const char *what) {
    if (got != want) {
        fprintf(stderr, "%s: returned %d, expected %d\n", what, got, want);
        ++g_failures;
    }
}

enum { B = 3, T = 2, H = 3, D = 6, HI = 3, DI = 5, K = 4, W = 5, R = 4, RH = 8 };

/* One batch: sequence 0 long, sequence 1 short, sequence 2 below one entry. */
static const int32_t kSeqLen[B] = {45, 11, 3};

static void run_dtype(int dtype) {
    const size_t es = dtype == ORACLE_F32 ? 4 : 2;
    int32_t seq_len[B], q_pos[B * T], win_pos0[B], win_rows[B];
    int n_max = 0;
    for (int b = 0; b < B; ++b) {
        seq_len[b] = kSeqLen[b];
        if (seq_len[b] / R > n_max) n_max = seq_len[b] / R;
        for (int t = 0; t < T; ++t) q_pos[b * T + t] = seq_len[b] - T + t; /* causal: the last T tokens */
        int first = q_pos[b * T] - W + 1;
        win_pos0[b] = first < 0 ? 0 : first;
        win_rows[b] = seq_len[b] - win_pos0[b];
    }
    void *q = values((size_t)B * T * H * D, dtype);
    void *q_idx = values((size_t)B * T * HI * DI, dtype);
    float *w = floats((size_t)B * T * HI, 0.f, 1.f);
    float *sink = floats(H, -1.f, 1.f);
    const void *k_idx[B], *kv[B], *v[B], *win[B], *win_v[B], *hkv[B];
    const uint8_t *k8[B];
    const float *k_scale[B];
    for (int b = 0; b < B; ++b) {
        const int n = seq_len[b] / R;
        k_idx[b] = values((size_t)n * DI, dtype);
        kv[b] = values((size_t)n * D, dtype);
        v[b] = values((size_t)n * D, dtype);
        win[b] = values((size_t)win_rows[b] * D, dtype);
        win_v[b] = values((size_t)win_rows[b] * D, dtype);
        hkv[b] = values((size_t)(seq_len[b] / RH) * D, dtype);
        uint8_t *c = xalloc((size_t)n * DI);
        for (int i = 0; i < n * DI; ++i) c[i] = (uint8_t)(uniform() * 256.0);
        k8[b] = c;
        k_scale[b] = floats((size_t)n, 0.01f, 0.1f);
    }
    const size_t Q = (size_t)B * T;
    float *scores = xalloc(Q * n_max * sizeof(float));
    int32_t *idx = xalloc(Q * K * sizeof(int32_t));
    int32_t *idx_wide = xalloc(Q * 16 * sizeof(int32_t));
    double *out = xalloc(Q * H * D * sizeof(double)), *lse = xalloc(Q * H * sizeof(double));
    for (int act = 0; act < 2; ++act) {
        expect(oracle_index_scores(B, T, HI, DI, R, act, dtype, q_idx, w, k_idx, seq_len, q_pos, n_max, scores), 0,
               "index_scores");
        expect(oracle_topk(B, T, R, K, scores, n_max, seq_len, q_pos, idx), 0, "topk");
        /* more entries asked for than any query sees: the rest is -1 */
        expect(oracle_topk(B, T, R, 16, scores, n_max, seq_len, q_pos, idx_wide), 0, "topk wide");
        for (size_t i = 0; i < Q * 16; ++i)
            if (idx_wide[i] < -1 || idx_wide[i] >= n_max) {
                fprintf(stderr, "topk wide: index %d out of range\n", idx_wide[i]);
                ++g_failures;
                break;
            }
        expect(oracle_sparse_mqa(B, T, H, D, K, W, R, dtype, 0.4, q, kv, NULL, win, NULL, win_pos0, win_rows, idx,
                                 seq_len, q_pos, sink, out, lse),
               0, "sparse_mqa (V = K)");
        expect(oracle_sparse_mqa(B, T, H, D, K, W, R, dtype, 0.4, q, kv, v, win, win_v, win_pos0, win_rows, idx,
                                 seq_len, q_pos, NULL, out, NULL),
               0, "sparse_mqa (separate V, no sink, no lse)");
        expect(oracle_csa_attention(B, T, H, D, HI, DI, K, W, R, act, dtype, 0.0, q, q_idx, w, k_idx, kv, v, win,
                                    win_v, win_pos0, win_rows, seq_len, q_pos, sink, n_max, scores, idx, out, lse),
               0, "csa_attention");
    }
    expect(oracle_hca_mqa(B, T, H, D, W, RH, dtype, 0.4, q, hkv, NULL, win, NULL, win_pos0, win_rows, seq_len,
                          q_pos, sink, out, lse),
           0, "hca_mqa");
    if (dtype == ORACLE_BF16) {
        uint8_t *q8 = xalloc(Q * HI * DI);
        for (size_t i = 0; i < Q * HI * DI; ++i) q8[i] = (uint8_t)(uniform() * 256.0);
        float *q_scale = floats(Q * HI, 0.01f, 0.1f);
        expect(oracle_index_scores_fp8(B, T, HI, DI, R, ORACLE_ACT_RELU, q8, q_scale, w, k8, k_scale, seq_len, q_pos,
                                       n_max, scores),
               0, "index_scores_fp8");
        free(q8);
        free(q_scale);
    }
    /* a window buffer that misses a window token */
    int32_t short_rows[B];
    memcpy(short_rows, win_rows, sizeof(short_rows));
    short_rows[0] -= 1;
    expect(oracle_sparse_mqa(B, T, H, D, K, W, R, dtype, 0.4, q, kv, NULL, win, NULL, win_pos0, short_rows, idx,
                             seq_len, q_pos, sink, out, lse),
           ORACLE_EWINDOW, "sparse_mqa (window short)");
    /* argument checks */
    expect(oracle_index_scores(B, T, HI, DI, R, 0, dtype, NULL, w, k_idx, seq_len, q_pos, n_max, scores),
           ORACLE_EINVAL, "index_scores (q_idx NULL)");
    expect(oracle_index_scores(B, T, HI, DI, 0, 0, dtype, q_idx, w, k_idx, seq_len, q_pos, n_max, scores),
           ORACLE_EINVAL, "index_scores (ratio 0)");
    expect(oracle_topk(B, T, R, 0, scores, n_max, seq_len, q_pos, idx), ORACLE_EINVAL, "topk (K = 0)");
    expect(oracle_sparse_mqa(B, T, H, 0, K, W, R, dtype, 0.4, q, kv, NULL, win, NULL, win_pos0, win_rows, idx,
                             seq_len, q_pos, sink, out, lse),
           ORACLE_EINVAL, "sparse_mqa (D = 0)");

    /* row-list attention: partials over two halves merged equal the whole */
    enum { N = 7 };
    const void *rows[N], *vrows[N];
    for (int i = 0; i < N; ++i) {
        rows[i] = values(D, dtype);
        vrows[i] = values(D, dtype);
    }
    double *m = xalloc(2 * H * sizeof(double)), *l = xalloc(2 * H * sizeof(double));
    double *o = xalloc(2 * H * D * sizeof(double));
    double *out1 = xalloc(H * D * sizeof(double)), *lse1 = xalloc(H * sizeof(double));
    double *out2 = xalloc(H * D * sizeof(double)), *lse2 = xalloc(H * sizeof(double));
    expect(oracle_attend_rows(H, D, dtype, 0.3, q, rows, vrows, N, sink, out1, lse1), 0, "attend_rows");
    expect(oracle_partial_rows(H, D, dtype, 0.3, q, rows, vrows, 3, m, l, o), 0, "partial_rows");
    expect(oracle_partial_rows(H, D, dtype, 0.3, q, rows + 3, vrows + 3, N - 3, m + H, l + H, o + H * D), 0,
           "partial_rows");
    expect(oracle_merge_partials(2, H, D, m, l, o, sink, out2, lse2), 0, "merge_partials");
    for (int i = 0; i < H * D; ++i)
        if (fabs(out1[i] - out2[i]) > 1e-12) {
            fprintf(stderr, "merged partials differ from the whole at %d\n", i);
            ++g_failures;
            break;
        }
    expect(oracle_attend_rows(H, D, dtype, 0.3, q, rows, NULL, 0, sink, out1, lse1), 0, "attend_rows (no rows)");
    for (int i = 0; i < N; ++i) {
        free((void *)rows[i]);
        free((void *)vrows[i]);
    }
    free(m), free(l), free(o), free(out1), free(lse1), free(out2), free(lse2);

    for (int b = 0; b < B; ++b) {
        free((void *)k_idx[b]), free((void *)kv[b]), free((void *)v[b]), free((void *)win[b]);
        free((void *)win_v[b]), free((void *)hkv[b]), free((void *)k8[b]), free((void *)k_scale[b]);
    }
    free(q), free(q_idx), free(w), free(sink), free(scores), free(idx), free(idx_wide), free(out), free(lse);
    (void)es;
}

static void run_compress(void) {
    enum { TOK = 21, HID = 16, OUT = 8, CR = 4, CW = 8, ROPE = 4 };
    uint16_t *x = values((size_t)TOK * HID, ORACLE_BF16);
    uint16_t *wkv = values((size_t)OUT * HID, ORACLE_BF16);
    uint16_t *wgate = values((size_t)OUT * HID, ORACLE_BF16);
    float *ape = floats((size_t)CW * OUT, -0.5f, 0.5f);
    float *gamma = floats(OUT, 0.5f, 1.5f);
    const int n_entries = TOK / CR;
    double *out = xalloc((size_t)n_entries * OUT * sizeof(double));
    for (int had = 0; had < 2; ++had)
        expect(oracle_compress(TOK, HID, OUT, CR, CW, ROPE, 160000.0, 1e-6, had, x, 0, wkv, wgate, ape, gamma, 0,
                               n_entries, out),
               0, "compress");
    /* x starting after an entry's window: its tokens are not supplied */
    expect(oracle_compress(TOK - 4, HID, OUT, CR, CW, ROPE, 160000.0, 1e-6, 0, x, 4, wkv, wgate, ape, gamma, 0, 1,
                           out),
           ORACLE_EWINDOW, "compress (window not supplied)");
    free(x), free(wkv), free(wgate), free(ape), free(gamma), free(out);
}

int main(void) {
    for (int64_t L = 0; L < 40; ++L)
        for (int64_t p = 0; p < L; ++p) {
            const int64_t n = oracle_visible_count(L, p, R);
            if (n < 0 || n > L / R) {
                fprintf(stderr, "visible_count(%lld, %lld) = %lld\n", (long long)L, (long long)p, (long long)n);
                ++g_failures;
            }
        }
    for (int c = 0; c < 256; ++c) {
        const double v = oracle_e4m3_value((uint8_t)c);
        if ((c & 0x7f) != 0x7f && !(fabs(v) <= 448.0)) {
            fprintf(stderr, "e4m3 code %d -> %g\n", c, v);
            ++g_failures;
        }
    }
    run_dtype(ORACLE_F32);
    run_dtype(ORACLE_BF16);
    run_compress();
    if (g_failures) {
        fprintf(stderr, "%d failures\n", g_failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
