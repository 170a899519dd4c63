// fp8 (OCP E4M3) indexer scorer with per-row scales ("DeepSeek-V4-Flash-0731"
// config table, quantization_config: fp8, E4M3; "DeepSeek-V4 Architecture
// Analysis", INNOVATIONS 1, indexer bullet: quantization-aware training).
#include "common.hpp"
#include "launch.hpp"
#include "scorer_common.hpp"

namespace csa {

// ---------------------------------------------------------------------------
// fp8 (OCP E4M3) decode scorer with per-row scales, HI = 64, DI = 128: the
// same organisation as the bf16 decode scorer on v_mfma_f32_16x16x32_fp8_fp8
// (A: 8 codes of head e's row per lane, B: 8 codes of entry e per lane).
// Keys are 128 bytes per entry, half the bf16 stream.  Scales are positive,
// so ReLU commutes with them: s_j = k_scale_j * sum_h (w_h q_scale_h)
// act(q8_h . k8_j); the head weights absorb the query scales once, and each
// stored score takes its entry's scale.  A wave-step is 64 entries (8 KiB,
// 1 KiB contiguous per load instruction), redistributed through a
// wave-private LDS block as in the bf16 kernel.  Unlike the bf16 kernel, the
// workgroup steps of a query are dealt round-robin to its workgroups: the
// contiguous stretches with a start barrier measured slower for these rows.
namespace {
constexpr int kF8WaveStep = 64;                        // entries per wave and step
constexpr int kF8WgStep = kScoreWaves * kF8WaveStep;   // entries per workgroup step
constexpr int kF8RowWords = 128 / 4 + 4;               // LDS row: 128 codes + 16 B pad
constexpr int kF8Depth = 2;                            // wave-steps of loads in flight
struct F8Raw {
    u32x4_t k[8];  // 64 rows x 128 bytes, 16 bytes per lane per load
    float ks;      // scale of the entry this lane stores
};
}  // namespace

template <int kAct, int kDepth>
__global__ __launch_bounds__(64 * kScoreWaves, 1) void index_scores_fp8_kernel(ScoreArgs a) {
    __shared__ __attribute__((aligned(16))) uint32_t kraw[kScoreWaves][kF8WaveStep * kF8RowWords];
    const int qi = blockIdx.y;
    const int b = qi / a.T;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int e = lane & 15, g = lane >> 4;

    int nvis = visible_entries(a.seq_len[b], a.q_pos[qi], a.ratio);
    nvis = nvis < a.n_max ? nvis : a.n_max;
    float *srow = a.scores + (size_t)qi * a.n_max;

    // A fragments: head 16*ht + e, codes 32s + 8g .. +8 for k-step s.
    uint64_t qa[4][4];
    const uint8_t *qb = (const uint8_t *)a.q_idx + (size_t)qi * kHI * kDI;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int s = 0; s < 4; ++s) qa[ht][s] = *(const uint64_t *)(qb + (16 * ht + e) * kDI + 32 * s + 8 * g);
    // weights of the C-tile rows this lane holds (head 16*ht + 4g + r), times the query-row scales
    float wr[4][4];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const size_t h = (size_t)qi * kHI + 16 * ht + 4 * g + r;
            wr[ht][r] = a.w[h] * a.q_scale[h];
        }

    const uint8_t *kb = (const uint8_t *)a.k_idx[b];
    const float *ksb = (const float *)a.k_scale[b];
    const int last = nvis > 0 ? nvis - 1 : 0;
    const int stride = gridDim.x * kF8WgStep;
    const int base0 = blockIdx.x * kF8WgStep + wave * kF8WaveStep;
    const int n_steps = base0 < a.n_max ? (a.n_max - base0 + stride - 1) / stride : 0;
    const int n_load = base0 < nvis ? (nvis - base0 + stride - 1) / stride : 0;

    auto load = [&](F8Raw &kr, int base) {  // unconditional, indices clamped into the visible rows
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int j = base + 8 * i + (lane >> 3);
            j = j < nvis ? j : last;
            kr.k[i] = __builtin_nontemporal_load(as_global<u32x4_t>(kb + (size_t)j * kDI + 16 * (lane & 7)));
        }
        int js = base + 16 * g + e;
        js = js < nvis ? js : last;
        kr.ks = ksb[js];
    };
    uint32_t *kw = kraw[wave];
    auto process = [&](F8Raw &kr, int base, bool live, int next) {
#pragma unroll
        for (int i = 0; i < 8; ++i) *(u32x4_t *)&kw[(8 * i + (lane >> 3)) * kF8RowWords + 4 * (lane & 7)] = kr.k[i];
        const float ks = kr.ks;
        load(kr, next);  // registers free again: the next loads go out before the math
        const int j = base + 16 * g + e;  // entry this lane stores
        float mine = 0.f;
#pragma unroll
        for (int et = 0; et < 4; ++et) {
            uint64_t kf[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) kf[s] = *(const uint64_t *)&kw[(16 * et + e) * kF8RowWords + 8 * s + 2 * g];
            f32x4_t acc[4];
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) {
                acc[ht] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)qa[ht][s], (long)kf[s], acc[ht], 0, 0,
                                                                        0);
            }
            float p = 0.f;
#pragma unroll
            for (int ht = 0; ht < 4; ++ht)
#pragma unroll
                for (int r = 0; r < 4; ++r) p = fmaf(wr[ht][r], index_act<kAct>(acc[ht][r]), p);
            p = sum_xor16(p);
            p = sum_xor32(p);
            if (g == et) mine = p;  // lane group g keeps column tile g
        }
        if (live && j < a.n_max) srow[j] = j < nvis ? ks * mine : -INFINITY;
    };

    if (n_load > 0) {
        // kDepth steps in flight, unrolled so no load sits behind a branch; steps past the
        // last one reload the last step and store nothing
        F8Raw kbuf[kDepth];
        auto step = [&](int k) { return base0 + (k < n_load ? k : n_load - 1) * stride; };
#pragma unroll
        for (int i = 0; i < kDepth; ++i) load(kbuf[i], step(i));
        for (int k = 0; k < n_load; k += kDepth) {
#pragma unroll
            for (int i = 0; i < kDepth; ++i) process(kbuf[i], step(k + i), k + i < n_load, step(k + i + kDepth));
        }
    }
    for (int k = n_load; k < n_steps; ++k) {  // steps past the visible entries: -inf
        const int j = base0 + k * stride + 16 * g + e;
        if (j < a.n_max) srow[j] = -INFINITY;
    }
}

hipError_t launch_index_scores_fp8(const ScoreArgs &a, hipStream_t stream) {
    const int Q = a.B * a.T;
    int per_query = (kTargetWgs + Q - 1) / Q;
    const int steps = (a.n_max + kF8WgStep - 1) / kF8WgStep;
    if (per_query > steps) per_query = steps;
    if (per_query < 1) per_query = 1;
    const dim3 grid(per_query, Q), block(64 * kScoreWaves);
    if (a.act == 0)
        hipLaunchKernelGGL((index_scores_fp8_kernel<0, kF8Depth>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((index_scores_fp8_kernel<1, kF8Depth>), grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace csa
