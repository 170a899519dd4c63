// Exercises the host side of the C ABI -- argument and shape checks,
// workspace sizing, status strings -- over valid and invalid sizes up to the
// documented limits.  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host (the library's sources compiled for
// the host only, so no kernel exists to launch): every call here returns
// before anything is enqueued.  Prints "ok" and exits 0 when every call
// returned the expected status.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "csa.h"

static int g_failures = 0;

static void expect(int got, int want, const char *what) {
    if (got != want) {
        std::fprintf(stderr, "%s: returned %d (%s), expected %d; last error: %s\n", what, got,
                     csa_status_string(got), want, csa_last_error());
        ++g_failures;
    }
}

static csa_dims decode_dims() {
    csa_dims d{};
    d.batch = 4;
    d.q_len = 1;
    d.n_heads = 64;
    d.head_dim = 512;
    d.index_heads = 64;
    d.index_dim = 128;
    d.topk = 512;
    d.window = 128;
    d.ratio = 4;
    d.max_entries = 262144;
    d.dtype = CSA_BF16;
    d.index_act = CSA_ACT_RELU;
    d.softmax_scale = 0.f;
    return d;
}

// Workspace sizes of every op for one shape: the expected status for the
// fused op, and monotone growth of the fused op's bytes with its parts.
static void sizes(const csa_dims &d, int want_fused, const char *what) {
    size_t fused = 0, part = 0;
    expect(csa_workspace_size(&d, CSA_OP_ATTENTION, &fused), want_fused, what);
    if (want_fused != CSA_OK) return;
    const int ops[] = {CSA_OP_INDEX_SCORES, CSA_OP_TOPK, CSA_OP_SPARSE_MQA, CSA_OP_HCA_MQA};
    for (int op : ops) {
        expect(csa_workspace_size(&d, op, &part), CSA_OK, what);
        if (op != CSA_OP_HCA_MQA && part > fused) {
            std::fprintf(stderr, "%s: op %d needs %zu bytes, more than the fused call's %zu\n", what, op, part, fused);
            ++g_failures;
        }
    }
    const size_t scores = (size_t)d.batch * d.q_len * (size_t)d.max_entries * 4;
    if (fused < scores) {
        std::fprintf(stderr, "%s: fused workspace %zu holds no score rows (%zu)\n", what, fused, scores);
        ++g_failures;
    }
}

int main() {
    if (csa_abi_version() != CSA_ABI_VERSION) {
        std::fprintf(stderr, "abi version mismatch\n");
        ++g_failures;
    }
    for (int s = -2; s < 10; ++s)
        if (!csa_status_string(s) || !std::strlen(csa_status_string(s))) ++g_failures;

    // shapes the kernels support, up to the documented limits
    csa_dims d = decode_dims();
    sizes(d, CSA_OK, "decode batch 4 x 262144");
    d.n_heads = 128;
    sizes(d, CSA_OK, "decode 128 heads");
    d = decode_dims();
    d.batch = 1;
    d.q_len = 2048;
    sizes(d, CSA_OK, "prefill 2048 x 262144");
    d = decode_dims();
    d.batch = 32;
    d.max_entries = 32768;
    sizes(d, CSA_OK, "decode batch 32");
    d = decode_dims();
    d.batch = 1 << 20;
    d.max_entries = 1 << 26;
    d.topk = 2048;
    d.window = 1 << 20;
    sizes(d, CSA_OK, "every limit at once");
    d = decode_dims();
    d.batch = 1;
    d.max_entries = 1;
    d.topk = 1;
    d.window = 1;
    sizes(d, CSA_OK, "one entry");
    for (int n = 1; n <= 70000; n = n * 3 + 1) {  // the selection's regimes (direct, histogram, lists)
        d = decode_dims();
        d.max_entries = n;
        for (int k : {1, 7, 512, 2048}) {
            d.topk = k;
            sizes(d, CSA_OK, "entry sweep");
        }
    }
    csa_dims f{};
    f.batch = 3;
    f.q_len = 5;
    f.n_heads = 5;
    f.head_dim = 24;
    f.index_heads = 3;
    f.index_dim = 16;
    f.topk = 7;
    f.window = 9;
    f.ratio = 4;
    f.max_entries = 50;
    f.dtype = CSA_F32;
    sizes(f, CSA_OK, "fp32 small");

    // invalid shapes
    struct Bad {
        const char *what;
        void (*edit)(csa_dims &);
        int want;
    } bad[] = {
        {"batch 0", [](csa_dims &x) { x.batch = 0; }, CSA_ERR_DIM},
        {"q_len negative", [](csa_dims &x) { x.q_len = -3; }, CSA_ERR_DIM},
        {"queries over the limit", [](csa_dims &x) { x.batch = INT_MAX; x.q_len = INT_MAX; }, CSA_ERR_DIM},
        {"ratio 0", [](csa_dims &x) { x.ratio = 0; }, CSA_ERR_DIM},
        {"max_entries 0", [](csa_dims &x) { x.max_entries = 0; }, CSA_ERR_DIM},
        {"max_entries over the limit", [](csa_dims &x) { x.max_entries = INT_MAX; }, CSA_ERR_DIM},
        {"unknown dtype", [](csa_dims &x) { x.dtype = 7; }, CSA_ERR_UNSUPPORTED},
        {"topk 0", [](csa_dims &x) { x.topk = 0; }, CSA_ERR_DIM},
        {"topk over the limit", [](csa_dims &x) { x.topk = 4096; }, CSA_ERR_DIM},
        {"window 0", [](csa_dims &x) { x.window = 0; }, CSA_ERR_DIM},
        {"window huge", [](csa_dims &x) { x.window = INT_MAX; }, CSA_ERR_DIM},
        {"scale negative", [](csa_dims &x) { x.softmax_scale = -1.f; }, CSA_ERR_DIM},
        {"scale NaN", [](csa_dims &x) { x.softmax_scale = std::nanf(""); }, CSA_ERR_DIM},
        {"scale inf", [](csa_dims &x) { x.softmax_scale = INFINITY; }, CSA_ERR_DIM},
        {"bf16 head_dim", [](csa_dims &x) { x.head_dim = 256; }, CSA_ERR_UNSUPPORTED},
        {"bf16 index_dim", [](csa_dims &x) { x.index_dim = 64; }, CSA_ERR_UNSUPPORTED},
        {"unknown act", [](csa_dims &x) { x.index_act = 5; }, CSA_ERR_UNSUPPORTED},
        {"heads 0", [](csa_dims &x) { x.n_heads = 0; }, CSA_ERR_DIM},
    };
    for (const Bad &b : bad) {
        d = decode_dims();
        b.edit(d);
        sizes(d, b.want, b.what);
    }
    size_t bytes = 1;
    d = decode_dims();
    expect(csa_workspace_size(&d, 99, &bytes), CSA_ERR_UNSUPPORTED, "unknown op");
    expect(csa_workspace_size(nullptr, CSA_OP_TOPK, &bytes), CSA_ERR_NULL, "dims NULL");
    expect(csa_workspace_size(&d, CSA_OP_TOPK, nullptr), CSA_ERR_NULL, "bytes NULL");

    // entry points: every check that returns before a launch
    d = decode_dims();
    alignas(256) static unsigned char buf[4096];
    void *p = buf;                  // a stand-in address, never dereferenced
    void *mis = buf + 2;            // misaligned
    const void *const *pp = (const void *const *)buf;
    const int32_t *ip = (const int32_t *)buf;
    const float *fp = (const float *)buf;
    float *fo = (float *)buf;
    int32_t *io = (int32_t *)buf;
    expect(csa_index_scores(&d, nullptr, fp, pp, ip, ip, fo, nullptr, 0, nullptr), CSA_ERR_NULL, "scores q_idx NULL");
    expect(csa_index_scores(&d, mis, fp, pp, ip, ip, fo, nullptr, 0, nullptr), CSA_ERR_ALIGN, "scores misaligned");
    expect(csa_topk_select(&d, fp, ip, ip, io, nullptr, 0, nullptr), CSA_ERR_WORKSPACE, "topk no workspace");
    expect(csa_topk_select(&d, fp, ip, ip, io, p, 16, nullptr), CSA_ERR_WORKSPACE, "topk small workspace");
    expect(csa_topk_select(&d, fp, ip, nullptr, io, p, 16, nullptr), CSA_ERR_NULL, "topk q_pos NULL");
    expect(csa_sparse_mqa_decode(&d, p, pp, nullptr, ip, pp, nullptr, ip, ip, ip, ip, fp, fo, fo, p, 16, nullptr),
           CSA_ERR_WORKSPACE, "sparse small workspace");
    expect(csa_sparse_mqa_decode(&d, p, pp, nullptr, ip, pp, nullptr, ip, ip, ip, ip, nullptr, fo, fo, p, 16,
                                 nullptr),
           CSA_ERR_NULL, "sparse sink NULL");
    expect(hca_mqa_decode(&d, p, pp, nullptr, pp, nullptr, ip, ip, ip, ip, fp, (float *)mis, fo, p, 16, nullptr),
           CSA_ERR_ALIGN, "hca out misaligned");
    expect(csa_attention(&d, p, p, fp, pp, pp, nullptr, pp, nullptr, ip, ip, ip, ip, fp, fo, fo, nullptr, nullptr,
                         p, 16, nullptr),
           CSA_ERR_WORKSPACE, "attention small workspace");
    expect(csa_attention(&d, p, nullptr, fp, pp, pp, nullptr, pp, nullptr, ip, ip, ip, ip, fp, fo, fo, nullptr,
                         nullptr, p, 16, nullptr),
           CSA_ERR_NULL, "attention q_idx NULL");
    // the fp8 index path: sizes, its own checks
    d = decode_dims();
    expect(csa_workspace_size(&d, CSA_OP_ATTENTION_FP8, &bytes), CSA_OK, "fp8 fused sizes");
    d.dtype = CSA_F32;
    expect(csa_workspace_size(&d, CSA_OP_ATTENTION_FP8, &bytes), CSA_ERR_UNSUPPORTED, "fp8 fused, fp32 attention");
    d = decode_dims();
    d.index_dim = 64;
    expect(csa_workspace_size(&d, CSA_OP_ATTENTION_FP8, &bytes), CSA_ERR_UNSUPPORTED, "fp8 fused, index_dim 64");
    d = decode_dims();
    const uint8_t *q8 = (const uint8_t *)buf;
    expect(csa_attention_fp8(&d, p, q8, nullptr, fp, pp, pp, pp, nullptr, pp, nullptr, ip, ip, ip, ip, fp, fo, fo,
                             nullptr, nullptr, p, 1u << 30, nullptr),
           CSA_ERR_NULL, "fp8 fused q_scale NULL");
    expect(csa_attention_fp8(&d, p, q8, fp, fp, pp, pp, pp, nullptr, pp, nullptr, ip, ip, ip, ip, fp, fo, fo, nullptr,
                             nullptr, p, 16, nullptr),
           CSA_ERR_WORKSPACE, "fp8 fused small workspace");
    d.q_len = 2048;
    d.batch = 1;
    sizes(d, CSA_OK, "prefill sizes before the fp8 ones");
    expect(csa_workspace_size(&d, CSA_OP_ATTENTION_FP8, &bytes), CSA_OK, "fp8 fused prefill sizes");
    d = decode_dims();
    d.batch = 1 << 20;  // far beyond the static work area
    expect(csa_attention_noalloc(&d, p, p, fp, pp, pp, nullptr, pp, nullptr, ip, ip, ip, ip, fp, fo, fo, nullptr,
                                 nullptr, nullptr),
           CSA_ERR_WORKSPACE, "noalloc over its limit");
    d.batch = 0;
    expect(csa_attention_noalloc(&d, p, p, fp, pp, pp, nullptr, pp, nullptr, ip, ip, ip, ip, fp, fo, fo, nullptr,
                                 nullptr, nullptr),
           CSA_ERR_DIM, "noalloc batch 0");

    // compressor
    csa_compress_dims c{};
    c.tokens = 4096;
    c.hidden = 4096;
    c.out_dim = 512;
    c.ratio = 4;
    c.window = 8;
    c.rope_dims = 64;
    c.hadamard = 0;
    c.first_entry = 2;
    c.n_entries = 1000;
    c.pos0 = 0;
    c.rope_theta = 160000.f;
    c.rms_eps = 1e-6f;
    expect(csa_compress_workspace_size(&c, &bytes), CSA_OK, "compress sizes");
    csa_compress_dims cb = c;
    cb.first_entry = INT_MAX / 2;
    cb.n_entries = INT_MAX / 2;
    expect(csa_compress_workspace_size(&cb, &bytes), CSA_ERR_DIM, "compress positions overflow");
    cb = c;
    cb.pos0 = 100;
    expect(csa_compress_workspace_size(&cb, &bytes), CSA_ERR_DIM, "compress window not covered");
    cb = c;
    cb.out_dim = 100;
    expect(csa_compress_workspace_size(&cb, &bytes), CSA_ERR_UNSUPPORTED, "compress out_dim");
    cb = c;
    cb.rope_dims = 3;
    expect(csa_compress_workspace_size(&cb, &bytes), CSA_ERR_DIM, "compress odd rope dims");
    expect(csa_compress(&c, p, p, p, fp, fp, p, nullptr, 0, nullptr), CSA_ERR_WORKSPACE, "compress no workspace");
    expect(csa_compress(&c, mis, p, p, fp, fp, p, p, 1u << 30, nullptr), CSA_ERR_ALIGN, "compress x misaligned");

    if (g_failures) {
        std::fprintf(stderr, "%d failures\n", g_failures);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
