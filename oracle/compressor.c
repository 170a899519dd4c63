/*
 * CPU oracle for the KV / index-key compressor -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain scalar loops in float64 following the definitions in oracle.h
 * (readings R8-R12).  Shares nothing with the HIP path.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static double bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* R12: Sylvester Hadamard matrix entry H[i][j] = (-1)^popcount(i & j). */
static double hadamard_entry(int i, int j) {
    return (__builtin_popcount((unsigned)(i & j)) & 1) ? -1.0 : 1.0;
}

int oracle_compress(int tokens, int hidden, int out_dim, int ratio, int window, int rope_dims,
                    double rope_theta, double eps, int hadamard, const uint16_t *x, int pos0,
                    const uint16_t *wkv, const uint16_t *wgate, const float *ape, const float *gamma,
                    int first_entry, int n_entries, double *out) {
    if (tokens <= 0 || hidden <= 0 || out_dim <= 0 || ratio <= 0 || window < ratio || n_entries <= 0 ||
        first_entry < 0 || rope_dims < 0 || rope_dims > out_dim || (rope_dims & 1) || eps <= 0.0)
        return ORACLE_EINVAL;
    if (hadamard && (out_dim & (out_dim - 1))) return ORACLE_EINVAL;
    if (!x || !wkv || !wgate || !ape || !gamma || !out) return ORACLE_EINVAL;
    for (int i = 0; i < n_entries; ++i) { /* R8: every existing window token must be supplied */
        const long e = first_entry + i, last = (long)ratio * e + ratio - 1;
        long first = last - window + 1;
        if (first < 0) first = 0;
        if (first < pos0 || last >= (long)pos0 + tokens) return ORACLE_EWINDOW;
    }
    double *kv = malloc(sizeof(double) * (size_t)window * out_dim);
    double *g = malloc(sizeof(double) * (size_t)window * out_dim);
    double *c = malloc(sizeof(double) * (size_t)out_dim);
    double *y = malloc(sizeof(double) * (size_t)out_dim);
    if (!kv || !g || !c || !y) {
        free(kv), free(g), free(c), free(y);
        return ORACLE_ENOMEM;
    }
    for (int i = 0; i < n_entries; ++i) {
        const long e = first_entry + i, last = (long)ratio * e + ratio - 1, start = last - window + 1;
        /* R9: per-token projections and gate logits (+ position-in-window embedding) */
        int n = 0;
        for (long t = start; t <= last; ++t) {
            if (t < 0) continue; /* no token before the sequence start */
            const int slot = (int)(t - start);
            const uint16_t *xt = x + (size_t)(t - pos0) * hidden;
            for (int d = 0; d < out_dim; ++d) {
                double a = 0.0, b = 0.0;
                for (int h = 0; h < hidden; ++h) {
                    const double xv = bf16_value(xt[h]);
                    a += bf16_value(wkv[(size_t)d * hidden + h]) * xv;
                    b += bf16_value(wgate[(size_t)d * hidden + h]) * xv;
                }
                kv[(size_t)n * out_dim + d] = a;
                g[(size_t)n * out_dim + d] = b + (double)ape[(size_t)slot * out_dim + d];
            }
            ++n;
        }
        /* softmax over the window's tokens, per output dim; weighted sum of kv */
        for (int d = 0; d < out_dim; ++d) {
            double m = -INFINITY, z = 0.0, s = 0.0;
            for (int k = 0; k < n; ++k) m = fmax(m, g[(size_t)k * out_dim + d]);
            for (int k = 0; k < n; ++k) {
                const double p = exp(g[(size_t)k * out_dim + d] - m);
                z += p;
                s += p * kv[(size_t)k * out_dim + d];
            }
            c[d] = s / z;
        }
        /* R10: RMSNorm with learned weight */
        double ms = 0.0;
        for (int d = 0; d < out_dim; ++d) ms += c[d] * c[d];
        ms /= out_dim;
        const double inv = 1.0 / sqrt(ms + eps);
        for (int d = 0; d < out_dim; ++d) c[d] = c[d] * inv * (double)gamma[d];
        /* R11: RoPE on the trailing rope_dims dims, pairs (2k, 2k+1), position ratio * e */
        const int r0 = out_dim - rope_dims;
        for (int k = 0; k < rope_dims / 2; ++k) {
            const double ang = (double)(ratio * e) * pow(rope_theta, -2.0 * k / rope_dims);
            const double a = c[r0 + 2 * k], b = c[r0 + 2 * k + 1];
            c[r0 + 2 * k] = a * cos(ang) - b * sin(ang);
            c[r0 + 2 * k + 1] = a * sin(ang) + b * cos(ang);
        }
        /* R12: normalized Hadamard rotation of the whole vector */
        if (hadamard) {
            const double sc = 1.0 / sqrt((double)out_dim);
            for (int a = 0; a < out_dim; ++a) {
                double s = 0.0;
                for (int b = 0; b < out_dim; ++b) s += hadamard_entry(a, b) * c[b];
                y[a] = s * sc;
            }
            memcpy(c, y, sizeof(double) * (size_t)out_dim);
        }
        memcpy(out + (size_t)i * out_dim, c, sizeof(double) * (size_t)out_dim);
    }
    free(kv), free(g), free(c), free(y);
    return ORACLE_OK;
}
