// Kernel argument blocks and launchers (host side of the HIP path).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

struct ScoreArgs {
    const void *q_idx;          // [Q, HI, DI]
    const float *w;             // [Q, HI]
    const void *const *k_idx;   // [B] -> [N_b, DI]
    const int32_t *seq_len;     // [B]
    const int32_t *q_pos;       // [Q]
    float *scores;              // [Q, n_max]
    int B, T, HI, DI, ratio, act, n_max;
    // optional top-k key-histogram windows written by the bf16 kernel (null: skip),
    // one window per scorer workgroup of a query
    int32_t *win_hdr;           // [Q, n_win]
    uint32_t *win_cnt;          // [Q, n_win, kTopkWin]
    int K;
    // optional emitted entries of each workgroup for the selection (em_cap 0: none)
    int em_cap;                 // entries per workgroup at most
    int32_t *em_hdr;            // [Q, n_win, 2]: cut bin, count
    uint32_t *em_key;           // [Q, n_win, em_cap]
    int32_t *em_idx;            // [Q, n_win, em_cap]
    // tiled scorer only: 1 = write no scores; each (query, entry chunk) region
    // gets the chunk's K best entries (K <= kSelKeepMax <= em_cap)
    int sel_stream;
    // fp8 (E4M3) index tensors: per-row scales (null for bf16 / fp32)
    const float *q_scale;       // [Q, HI]
    const void *const *k_scale; // [B] -> [N_b] float
};

hipError_t launch_index_scores(const ScoreArgs &a, int dtype, hipStream_t stream);
// fp8 (E4M3) index queries and keys with per-row scales, HI = 64, DI = 128
// (histogram windows and emitted entries as for the bf16 decode scorer)
hipError_t launch_index_scores_fp8(const ScoreArgs &a, hipStream_t stream);

int score_workgroups(int n_max, int n_queries);  // bf16 scorer workgroups per query (even split)
// Decode-scorer geometry for the fused call: workgroups (= histogram windows
// and emitted regions) per query, emitted entries per region (0: none)
struct DecodeGeom {
    int n_win, em_cap, step;
};
DecodeGeom decode_geom(bool fp8, int n_max, int n_queries, int K);
// many queries per sequence: the GEMM-tiled scorer
bool score_uses_tiles(int dtype, int T);
// histogram windows per query the tiled scorer can write (its entry chunks), 0 if it cannot
int tiled_windows(int B, int T, int n_max);
// entries per (query, chunk) region handed to the selection after the tiled scorer, 0 if it cannot
int tiled_emit_cap(int B, int T, int n_max, int K);
// entries per chunk of the tiled scorer (its histogram windows' spans)
int tiled_chunk_entries(int B, int T, int n_max);

constexpr int kTopkSmallMax = 4096;       // rows up to this length: one workgroup, row kept in LDS
constexpr int kTopkOneKernelMax = 65536;  // rows up to this length: threshold+scan+select in one kernel
constexpr int kTopkBins = 4096;           // key histogram (top 12 key bits)
constexpr int kTopkWin = 32;              // histogram window kept per workgroup (4 octaves)
constexpr int kTopkCand = 8192;           // candidates held in LDS by the selecting workgroup
constexpr int kTopkMaxK = 2048;
constexpr int kTopkAuxChunk = 2048;       // scores per workgroup in the histogram and filter kernels
constexpr int kFltAboveCap = 64;          // per filter workgroup: entries above the threshold bin
constexpr int kFltCandCap = 256;          // per filter workgroup: candidates inside it
constexpr int kFltRegionWords = 2 + kFltAboveCap + 2 * kFltCandCap;
constexpr int kTopkManyQueries = 256;     // from this many queries on: one selecting workgroup per query
constexpr int kTopkMaxRegions = 256;      // emitted regions (decode-scorer workgroups) per query at most
constexpr int kTopkMaxSlots = 8192;       // emitted slots (regions x entries per region) per query at most
constexpr int kSelKeepMax = 512;         // K at most for the tiled scorer's streaming selection
constexpr int kSelChunkMax = 65536;      // entries per chunk at most for it (16-bit offsets)

struct TopkArgs {
    const float *scores;        // [Q, n_max]
    const int32_t *seq_len;     // [B]
    const int32_t *q_pos;       // [Q]
    int32_t *idx;               // [Q, K]
    int B, T, ratio, K, n_max;
    // scratch inside the caller's workspace (rows longer than kTopkSmallMax)
    int n_win;                  // histogram windows per query
    int hist_chunk;             // entries per window when the top-k builds its own histograms
    int32_t *win_hdr;           // [Q, n_win]
    uint32_t *win_cnt;          // [Q, n_win, kTopkWin]
    uint32_t *bin;              // [Q] threshold bin (long rows)
    uint32_t *flt;              // [Q, n_flt, kFltRegionWords] per-filter-workgroup lists (long rows)
    // the scorer's emitted entries, one region per window (em_cap 0: not used);
    // em_chunk > 0: the top-k emits the regions itself, one per window of
    // em_chunk entries, from the scores (after the tiled scorer)
    int em_cap, em_chunk;
    // 1: each region holds its chunk's K best entries (the tiled scorer's
    // streaming selection, no scores written); the threshold comes from the slots
    int em_stream;
    int32_t *em_hdr;            // [Q, n_win, 2]
    uint32_t *em_key;           // [Q, n_win, em_cap]
    int32_t *em_idx;            // [Q, n_win, em_cap]
};

// n_win: windows per query (scorer workgroups per query in the fused path, else 0 = own histogram kernel);
// em_cap: entries per window region the scorer emits (0: none)
size_t topk_workspace_bytes(int n_queries, int K, int n_max, int n_win, int em_cap = 0);
void topk_carve(TopkArgs &a, void *ws, int n_queries, int n_win, int em_cap = 0);
// hist_done: the scorer already wrote the histogram windows (fused path)
hipError_t launch_topk(const TopkArgs &a, hipStream_t stream, bool hist_done = false);
bool topk_uses_histogram(int n_max);

struct MqaArgs {
    const void *q;                  // [Q, H, D]
    const void *const *kv;          // [B] -> [N_b, D]
    const void *const *v;           // [B] -> [N_b, D] or null (V = K)
    const int32_t *topk_idx;        // [Q, K] or null (dense: every visible entry)
    const void *const *win;         // [B] -> [win_rows_b, D]
    const void *const *win_v;       // or null
    const int32_t *win_pos0;        // [B]
    const int32_t *win_rows;        // [B]
    const int32_t *seq_len;         // [B]
    const int32_t *q_pos;           // [Q]
    const float *sink;              // [H]
    float *out;                     // [Q, H, D]
    float *lse;                     // [Q, H] or null
    void *part_o;                   // [Q, S, 8, 8, 64] 16-byte fp16 vectors: split partials O / l
    float *part_ml;                 // [Q, S, H, 4]: m, l, inverse scales of the two dim halves' O / l
    int B, T, H, D, K, W, ratio;
    int n_splits, n_tiles;          // splits per query; kTile-row tiles of the longest row list
    float scale;                    // softmax scale (natural units)
};

// Split plan for the bf16 split-K kernel: max_rows = largest row count of a query.
// Split s of a query takes tiles [s * n_tiles / n_splits, (s + 1) * n_tiles / n_splits).
void mqa_plan(int n_queries, int max_rows, int *n_splits, int *n_tiles);
size_t mqa_workspace_bytes(int dtype, int n_queries, int H, int D, int max_rows);
void mqa_carve(MqaArgs &a, void *ws, int n_queries);
hipError_t launch_mqa(const MqaArgs &a, int dtype, hipStream_t stream);

struct CompressArgs {
    const void *x;              // [tokens, hidden] bf16, token 0 at raw position pos0
    const void *wkv, *wgate;    // [out_dim, hidden] bf16
    const float *ape;           // [window, out_dim]
    const float *gamma;         // [out_dim]
    void *out;                  // [n_entries, out_dim] bf16
    float *part;                // [n_splits, tokens, 2 * out_dim] fp32 projections (workspace)
    int tokens, hidden, out_dim, ratio, window, rope_dims, hadamard, first_entry, n_entries, pos0, n_splits;
    float rope_theta, rms_eps;
    double rope_ln_theta;       // ln(rope_theta), worked out on the host in float64
};
int compress_splits(int tokens, int hidden, int out_dim);  // K splits of the projection
hipError_t launch_compress(CompressArgs a, hipStream_t stream);

}  // namespace csa
