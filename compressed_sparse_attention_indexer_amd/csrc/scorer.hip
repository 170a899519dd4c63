// Indexer scorer: s[q, j] = sum_h w[q,h] * act(q_idx[q,h,:] . k_idx_b[j,:]).
// The indexer compares each query against every compressed entry with a
// dot product per indexer head and weights the heads by per-query importance
// weights ("DeepSeek-V4 Architecture Analysis", INNOVATIONS 1, indexer bullet;
// DeepSeek-V4-Flash config: index_n_heads 64, index_head_dim 128).
#include "common.hpp"
#include "launch.hpp"
#include "topk_hist.hpp"

namespace csa {

// ---------------------------------------------------------------------------
// fp32 VALU kernel for small shapes (fixture).  One thread per entry, the
// query's index vectors and weights staged in LDS.
__global__ __launch_bounds__(256) void index_scores_f32_kernel(ScoreArgs a) {
    extern __shared__ float smem[];
    float *sq = smem;                           // [HI*DI]
    float *sw = smem + a.HI * a.DI;             // [HI]
    const int qi = blockIdx.y;
    const int b = qi / a.T;
    const float *qsrc = (const float *)a.q_idx + (size_t)qi * a.HI * a.DI;
    for (int i = threadIdx.x; i < a.HI * a.DI; i += blockDim.x) sq[i] = qsrc[i];
    for (int i = threadIdx.x; i < a.HI; i += blockDim.x) sw[i] = a.w[(size_t)qi * a.HI + i];
    __syncthreads();
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= a.n_max) return;
    int nvis = visible_entries(a.seq_len[b], a.q_pos[qi], a.ratio);
    nvis = nvis < a.n_max ? nvis : a.n_max;
    float *dst = a.scores + (size_t)qi * a.n_max + j;
    if (j >= nvis) {
        *dst = -INFINITY;
        return;
    }
    const float *kr = (const float *)a.k_idx[b] + (size_t)j * a.DI;
    float s = 0.f;
    for (int h = 0; h < a.HI; ++h) {
        float dot = 0.f;
        for (int d = 0; d < a.DI; ++d) dot = fmaf(sq[h * a.DI + d], kr[d], dot);
        const float act = a.act == 0 ? fmaxf(dot, 0.f) : dot;
        s = fmaf(sw[h], act, s);
    }
    *dst = s;
}

// ---------------------------------------------------------------------------
// bf16 MFMA decode scorer, HI = 64 heads, DI = 128.
//
// Per wave and step: 32 entries (two 16-entry column tiles) x 64 heads (four
// 16-head row tiles) x 128 dims (four k-steps of 32) on
// v_mfma_f32_16x16x32_bf16.  A = index query (heads x dims, resident in
// registers), B = index keys (dims x entries) loaded straight from HBM into
// registers with nontemporal loads, one step ahead of the step being
// computed.  Lane (e, g) of a tile holds dims [32s + 8g, 32s + 8g + 8) of
// entry e for k-step s, so each load instruction reads 64 contiguous bytes of
// every entry it touches.  The C tile gives each lane 4 heads of one entry;
// the weighted activation sum over those heads is done in registers and the 4
// lane groups are summed with two cross-lane adds.
//
// Launch shape: about one 4-wave workgroup per CU.  A workgroup-step covers
// 128 entries (32 KiB of keys); the steps of a query are dealt round-robin to
// its workgroups, so the workgroups in flight read neighbouring memory (the
// pattern that streams HBM fastest on this part).  Optionally each workgroup
// also histograms the keys of the scores it writes, for the top-k.
namespace {
constexpr int kHI = 64;
constexpr int kDI = 128;
constexpr int kScoreWaves = 4;
constexpr int kWaveStep = 32;                         // entries per wave and step
constexpr int kWgStep = kScoreWaves * kWaveStep;      // entries per workgroup step
constexpr int kTargetWgs = 256;                       // about one workgroup per CU
constexpr int kScoreDepth = 2;                        // key steps in flight per wave
typedef bf16x8_t KeyFrag[2][4];
}  // namespace

template <int kAct, bool kHist, int kDepth>
__global__ __launch_bounds__(64 * kScoreWaves, 1) void index_scores_bf16_kernel(ScoreArgs a) {
    __shared__ uint32_t lh[kHist ? kTopkBins : 1];
    __shared__ int s_red[4];
    const int qi = blockIdx.y;
    const int b = qi / a.T;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int e = lane & 15;   // entry (B column) / head row (A row) within a tile
    const int g = lane >> 4;   // dim group within a k-step

    int nvis = visible_entries(a.seq_len[b], a.q_pos[qi], a.ratio);
    nvis = nvis < a.n_max ? nvis : a.n_max;
    const bool with_hist = kHist && nvis > a.K;  // same for the whole workgroup
    if (with_hist) {
        for (int i = threadIdx.x; i < kTopkBins; i += 64 * kScoreWaves) lh[i] = 0u;
        __syncthreads();
    }
    float *srow = a.scores + (size_t)qi * a.n_max;

    // A fragments: head 16*ht + e, dims 32s + 8g .. +8 for k-step s.
    bf16x8_t qa[4][4];
    const uint16_t *qb = (const uint16_t *)a.q_idx + (size_t)qi * kHI * kDI;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            qa[ht][s] = *(const bf16x8_t *)(qb + (16 * ht + e) * kDI + 32 * s + 8 * g);
    // Importance weights of the C-tile rows this lane holds: head 16*ht + 4g + r.
    float wr[4][4];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int r = 0; r < 4; ++r) wr[ht][r] = a.w[(size_t)qi * kHI + 16 * ht + 4 * g + r];

    const uint16_t *kb = (const uint16_t *)a.k_idx[b];
    const int last = nvis > 0 ? nvis - 1 : 0;
    // step k of this wave starts at entry base0 + k * stride
    const int stride = gridDim.x * kWgStep;
    const int base0 = blockIdx.x * kWgStep + wave * kWaveStep;
    const int n_steps = base0 < a.n_max ? (a.n_max - base0 + stride - 1) / stride : 0;
    // steps that hold a visible entry come first: 0 .. n_load-1
    const int n_load = base0 < nvis ? (nvis - base0 + stride - 1) / stride : 0;

    // Every load is unconditional (indices clamped into the visible rows) so
    // the loop body is straight-line code and the compiler can wait for one
    // step's loads while the next step's are still in flight.
    auto load = [&](KeyFrag &kf, int base) {
#pragma unroll
        for (int et = 0; et < 2; ++et) {
            int j = base + 16 * et + e;
            j = j < nvis ? j : last;
            const gptr<bf16x8_t> kr = as_global<bf16x8_t>(kb + (size_t)j * kDI + 8 * g);
#pragma unroll
            for (int s = 0; s < 4; ++s) kf[et][s] = __builtin_nontemporal_load(kr + 4 * s);
        }
    };
    // `live`: the step exists (a clamped re-run of the last step stores nothing)
    auto process = [&](const KeyFrag &kf, int base, bool live) {
        const int j = base + 16 * g + e;  // entry this lane stores (g < 2)
        float part[2];
#pragma unroll
        for (int et = 0; et < 2; ++et) {
            f32x4_t acc[4];
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) {
                acc[ht] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ht][s], kf[et][s], acc[ht], 0, 0, 0);
            }
            float p = 0.f;
#pragma unroll
            for (int ht = 0; ht < 4; ++ht)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float x = acc[ht][r];
                    p = fmaf(wr[ht][r], kAct == 0 ? fmaxf(x, 0.f) : x, p);
                }
            p += __shfl_xor(p, 16);
            p += __shfl_xor(p, 32);
            part[et] = p;
        }
        // Lanes of group g < 2 store column tile g: 32 consecutive scores.
        const float sv = j < nvis ? (g == 0 ? part[0] : part[1]) : -INFINITY;
        if (live && g < 2 && j < a.n_max) srow[j] = sv;
        if (with_hist) lds_hist_add(lh, order_key(sv) >> 20, live && g < 2 && j < nvis);
    };

    if (n_load > 0) {
        // Software pipeline kDepth steps deep, unrolled by kDepth so that no
        // load sits behind a branch: while step k computes, the loads of steps
        // k+1 .. k+kDepth-1 are in flight.  Steps past the last one reload the
        // last step and store nothing.
        KeyFrag kbuf[kDepth];
        auto step = [&](int k) { return base0 + (k < n_load ? k : n_load - 1) * stride; };
#pragma unroll
        for (int i = 0; i < kDepth; ++i) load(kbuf[i], step(i));
        for (int k = 0; k < n_load; k += kDepth) {
#pragma unroll
            for (int i = 0; i < kDepth; ++i) {
                process(kbuf[i], step(k + i), k + i < n_load);
                load(kbuf[i], step(k + i + kDepth));
            }
        }
    }
    for (int k = n_load; k < n_steps; ++k) {  // steps past the visible entries: -inf
        const int j = base0 + k * stride + 16 * g + e;
        if (g < 2 && j < a.n_max) srow[j] = -INFINITY;
    }
    if (with_hist) {
        const size_t w = (size_t)qi * gridDim.x + blockIdx.x;
        hist_window_store(lh, a.win_hdr + w, a.win_cnt + w * kTopkWin, s_red);
    }
}

hipError_t launch_index_scores(const ScoreArgs &a, int dtype, hipStream_t stream) {
    const int Q = a.B * a.T;
    if (dtype == kF32) {
        dim3 grid((a.n_max + 255) / 256, Q);
        const size_t lds = sizeof(float) * (size_t)(a.HI * a.DI + a.HI);
        hipLaunchKernelGGL(index_scores_f32_kernel, grid, dim3(256), lds, stream, a);
        return hipGetLastError();
    }
    dim3 grid(score_workgroups(a.n_max, Q), Q);
    dim3 block(64 * kScoreWaves);
    const bool hist = a.win_hdr != nullptr;
    if (a.act == 0) {
        if (hist)
            hipLaunchKernelGGL((index_scores_bf16_kernel<0, true, kScoreDepth>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((index_scores_bf16_kernel<0, false, kScoreDepth>), grid, block, 0, stream, a);
    } else {
        if (hist)
            hipLaunchKernelGGL((index_scores_bf16_kernel<1, true, kScoreDepth>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((index_scores_bf16_kernel<1, false, kScoreDepth>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

int score_workgroups(int n_max, int n_queries) {
    // about one workgroup per CU over the launch, at most one per workgroup step
    int per_query = (kTargetWgs + n_queries - 1) / n_queries;
    const int steps = (n_max + kWgStep - 1) / kWgStep;
    if (per_query > steps) per_query = steps;
    return per_query < 1 ? 1 : per_query;
}

}  // namespace csa
