// fp8 (OCP E4M3) indexer scorer with per-row scales ("DeepSeek-V4-Flash-0731"
// config table, quantization_config: fp8, E4M3; "DeepSeek-V4 Architecture
// Analysis", INNOVATIONS 1, indexer bullet: quantization-aware training).
#include "common.hpp"
#include "launch.hpp"
#include "topk_hist.hpp"
#include "scorer_common.hpp"

namespace csa {

typedef int i32x8_t __attribute__((ext_vector_type(8)));  // 32 fp8 codes, an f8f6f4 MFMA operand

// ---------------------------------------------------------------------------
// fp8 (OCP E4M3) decode scorer with per-row scales, HI = 64, DI = 128: the
// organisation of the bf16 decode scorer on gfx950's
// v_mfma_f32_16x16x128_f8f6f4 (both operands E4M3, no block scales), one
// instruction per 16 heads x 16 entries x all 128 dims: lane (e, g) holds
// codes 32g .. 32g + 31 of head e's row (A) and of entry e's row (B).  A and B
// take their codes in the same lane positions, so the sum runs over every dim
// once whatever order the instruction adds them in.  Against four
// v_mfma_f32_16x16x32_fp8_fp8 per tile: 31.5 -> 29.3 us for batch 4 x 262,144
// entries.
// Keys are 128 bytes per entry, half the bf16 stream.  Scales are positive,
// so ReLU commutes with them: s_j = k_scale_j * sum_h (w_h q_scale_h)
// act(q8_h . k8_j); the head weights absorb the query scales once, and each
// stored score takes its entry's scale.  A wave-step is 64 entries (8 KiB,
// 1 KiB contiguous per load instruction), redistributed through a
// wave-private LDS block; every lane stores one score per step.  As in the
// bf16 kernel, each workgroup streams one contiguous stretch of its query's
// entries, its waves lined up by a barrier after their first loads, and it
// can build the selection's histogram window and emitted entries as it goes.
namespace {
constexpr int kF8WaveStep = 64;                        // entries per wave and step
constexpr int kF8WgStep = kFp8WgStep;                  // entries per workgroup step
constexpr int kF8RowWords = 128 / 4 + 4;               // LDS row: 128 codes + 16 B pad
constexpr int kF8Depth = 2;                            // wave-steps of loads in flight
struct F8Raw {
    u32x4_t k[8];  // 64 rows x 128 bytes, 16 bytes per lane per load
    float ks;      // scale of the entry this lane stores (scales read from global memory per step)
};
}  // namespace

// kLdsScale: the stretch's key scales are read into LDS once, before the key
// stream starts (the host picks it when every stretch fits kEmitMax entries).
// Read per step from global memory instead, next to the keys, the 4-byte scale
// loads and the score stores together made the compiler wait for every load
// in flight at each pass of the loop (vmcnt(0)), so the two steps in flight
// drained every other step: 27.8 against 24.3 us for the same loop without
// scales, without the MFMA work.
template <int kAct, bool kHist, bool kLdsScale, int kDepth>
__global__ __launch_bounds__(64 * kScoreWaves, 1) void index_scores_fp8_kernel(ScoreArgs a) {
    __shared__ uint32_t lh[kHist ? kTopkBins : 1];
    __shared__ uint32_t lkeys[kHist ? kEmitMax : 1];  // keys of this workgroup's stretch (emission)
    __shared__ float lks[kLdsScale ? kEmitMax : 1];   // key scales of this workgroup's stretch
    __shared__ __attribute__((aligned(16))) uint32_t kraw[kScoreWaves][kF8WaveStep * kF8RowWords];
    __shared__ int s_red[4];
    __shared__ int s_scan[4];  // the emission's scans (s_red may still be read after the window store)
    __shared__ int s_cut;
    // this workgroup's query, and its part of the query's entries (of n_parts)
    const int qi = blockIdx.y, part = blockIdx.x, n_parts = gridDim.x;
    const int b = qi / a.T;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int e = lane & 15, g = lane >> 4;

    int nvis = visible_entries(a.seq_len[b], a.q_pos[qi], a.ratio);
    nvis = nvis < a.n_max ? nvis : a.n_max;
    const bool with_hist = kHist && nvis > a.K;  // same for the whole workgroup
    float *srow = a.scores + (size_t)qi * a.n_max;

    i32x8_t qa[4];  // A fragments: head 16*ht + e, codes 32g .. 32g + 31
    const uint8_t *qb = (const uint8_t *)a.q_idx + (size_t)qi * kHI * kDI;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
        const u32x4_t lo = *(const u32x4_t *)(qb + (16 * ht + e) * kDI + 32 * g);
        const u32x4_t hi = *(const u32x4_t *)(qb + (16 * ht + e) * kDI + 32 * g + 16);
        qa[ht] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                         (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
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
    // Work split as in the bf16 kernel: the query's visible entries, in
    // workgroup steps of kF8WgStep, are cut into n_parts contiguous stretches;
    // wave w takes entries kF8WaveStep * w .. + kF8WaveStep - 1 of each step.
    const int vis_steps = (nvis + kF8WgStep - 1) / kF8WgStep;
    const int chunk = (vis_steps + n_parts - 1) / n_parts;
    const int s0 = part * chunk;
    const int n_load = vis_steps - s0 < chunk ? (vis_steps - s0 > 0 ? vis_steps - s0 : 0) : chunk;
    const int stride = kF8WgStep;
    const int base0 = s0 * kF8WgStep + wave * kF8WaveStep;
    // the host enables emission only when every stretch fits lkeys (checked here too)
    const bool emit = kHist && with_hist && a.em_cap > 0 && n_load * kF8WgStep <= kEmitMax;
    const int stretch0 = s0 * kF8WgStep;

    auto load = [&](F8Raw &kr, int base) {  // unconditional, indices clamped into the visible rows
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int j = base + 8 * i + (lane >> 3);
            j = j < nvis ? j : last;
            kr.k[i] = __builtin_nontemporal_load(as_global<u32x4_t>(kb + (size_t)j * kDI + 16 * (lane & 7)));
        }
        if (!kLdsScale) {
            int js = base + 16 * g + e;
            js = js < nvis ? js : last;
            kr.ks = ksb[js];
        }
    };
    uint32_t *kw = kraw[wave];
    int hmax = -1;  // highest histogram bin this thread added
    auto process = [&](F8Raw &kr, int base, bool live, int next) {
#pragma unroll
        for (int i = 0; i < 8; ++i) *(u32x4_t *)&kw[(8 * i + (lane >> 3)) * kF8RowWords + 4 * (lane & 7)] = kr.k[i];
        const int j = base + 16 * g + e;  // entry this lane stores
        const float ks = kLdsScale ? lks[j < nvis ? min(j - stretch0, kEmitMax - 1) : 0] : kr.ks;
        load(kr, next);  // registers free again: the next loads go out before the math
        float mine = 0.f;
        // all four column tiles' fragments read before the MFMAs (read per
        // tile, each tile's MFMAs waited out its reads' latency)
        i32x8_t kfs[4];
#pragma unroll
        for (int et = 0; et < 4; ++et) {
            const u32x4_t klo = *(const u32x4_t *)&kw[(16 * et + e) * kF8RowWords + 8 * g];
            const u32x4_t khi = *(const u32x4_t *)&kw[(16 * et + e) * kF8RowWords + 8 * g + 4];
            kfs[et] = i32x8_t{(int)klo[0], (int)klo[1], (int)klo[2], (int)klo[3],
                              (int)khi[0], (int)khi[1], (int)khi[2], (int)khi[3]};
        }
#pragma unroll
        for (int et = 0; et < 4; ++et) {
            const i32x8_t kf = kfs[et];
            // operand formats 0, 0: E4M3 x E4M3; scale operands 0: no block scaling
            const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
            f32x4_t acc[4];
#pragma unroll
            for (int ht = 0; ht < 4; ++ht)
                acc[ht] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[ht], kf, zero, 0, 0, 0, 0, 0, 0);
            float p = 0.f;
#pragma unroll
            for (int ht = 0; ht < 4; ++ht)
#pragma unroll
                for (int r = 0; r < 4; ++r) p = fmaf(wr[ht][r], index_act<kAct>(acc[ht][r]), p);
            p = sum_xor16(p);
            p = sum_xor32(p);
            if (g == et) mine = p;  // lane group g keeps column tile g
        }
        __builtin_amdgcn_sched_group_barrier(0x100, kLdsScale ? 9 : 8, 0);  // LDS reads (the scale's too)
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);                 // then the MFMAs
        const float sv = j < nvis ? ks * mine : -INFINITY;
        if (live && j < a.n_max) srow[j] = sv;
        if (with_hist) {
            const uint32_t key = order_key(sv);
            const uint32_t bin = key >> 20;
            const bool add = live && j < nvis;
            lds_hist_add(lh, bin, add);
            if (add) hmax = max(hmax, (int)bin);
            if (emit && add) lkeys[j - stretch0] = key;
        }
    };

    // kDepth steps in flight, unrolled so no load sits behind a branch; steps
    // past the last one reload the last step and store nothing.  The histogram
    // is cleared while the first loads are out, then the waves meet.
    F8Raw kbuf[kDepth];
    auto step = [&](int k) { return base0 + (k < n_load ? k : n_load - 1) * stride; };
    if (n_load > 0) {
#pragma unroll
        for (int i = 0; i < kDepth; ++i) load(kbuf[i], step(i));
    }
    // visible entries of this stretch: stretch0 .. stretch0 + n_st - 1
    int n_st = min(nvis, (s0 + n_load) * kF8WgStep) - stretch0;
    n_st = n_st > 0 ? n_st : 0;
    if (kLdsScale) {  // after the first key loads, so their latency covers these
        n_st = n_st < kEmitMax ? n_st : kEmitMax;  // the host's bound on the stretch makes this a no-op
        // indices past the stretch are clamped to its last entry: those lanes
        // read and write that entry's own scale again (no branch around a store)
        constexpr int kNT = 64 * kScoreWaves, kU = 16;
        for (int i0 = 0; i0 < n_st; i0 += kNT * kU) {
            float v[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int i = min(i0 + kNT * u + (int)threadIdx.x, n_st - 1);
                v[u] = ksb[stretch0 + i];
            }
#pragma unroll
            for (int u = 0; u < kU; ++u) lks[min(i0 + kNT * u + (int)threadIdx.x, n_st - 1)] = v[u];
        }
    }
    if (with_hist) {
        for (int i = threadIdx.x; i < kTopkBins; i += 64 * kScoreWaves) lh[i] = 0u;
    }
    __syncthreads();
    if (n_load > 0) {
        for (int k = 0; k < n_load; k += kDepth) {
#pragma unroll
            for (int i = 0; i < kDepth; ++i) process(kbuf[i], step(k + i), k + i < n_load, step(k + i + kDepth));
        }
    }
    const int all_steps = (a.n_max + kF8WgStep - 1) / kF8WgStep;
    for (int st = vis_steps + part; st < all_steps; st += n_parts) {  // steps past the visible entries
        const int j = st * kF8WgStep + wave * kF8WaveStep + 16 * g + e;
        if (j < a.n_max) srow[j] = -INFINITY;
    }
    if (with_hist) {
        const size_t w = (size_t)qi * n_parts + part;
        const int top = hist_window_store_top(lh, hmax, a.win_hdr + w, a.win_cnt + w * kTopkWin, s_red);
        decode_emission<64 * kScoreWaves>(a, lh, lkeys, emit, nvis, s0, n_load, kF8WgStep, w, top, s_scan, &s_cut);
    }
}


template <int kAct, bool kHist>
static void launch_fp8(const ScoreArgs &a, dim3 grid, dim3 block, bool lds_scale, hipStream_t stream) {
    if (lds_scale)
        hipLaunchKernelGGL((index_scores_fp8_kernel<kAct, kHist, true, kF8Depth>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((index_scores_fp8_kernel<kAct, kHist, false, kF8Depth>), grid, block, 0, stream, a);
}

hipError_t launch_index_scores_fp8(const ScoreArgs &a, hipStream_t stream) {
    const int Q = a.B * a.T;
    const int wgs = decode_score_workgroups(a.n_max, Q, kF8WgStep);
    const dim3 grid(wgs, Q), block(64 * kScoreWaves);
    const bool hist = a.win_hdr != nullptr;  // the caller sized the windows with decode_geom
    // every workgroup's stretch (at most ceil(steps / wgs) steps) fits the LDS scale buffer
    const int steps = (a.n_max + kF8WgStep - 1) / kF8WgStep;
    const bool lds_scale = (long)((steps + wgs - 1) / wgs) * kF8WgStep <= kEmitMax;
    if (a.act == 0) {
        if (hist) launch_fp8<0, true>(a, grid, block, lds_scale, stream);
        else launch_fp8<0, false>(a, grid, block, lds_scale, stream);
    } else {
        if (hist) launch_fp8<1, true>(a, grid, block, lds_scale, stream);
        else launch_fp8<1, false>(a, grid, block, lds_scale, stream);
    }
    return hipGetLastError();
}

}  // namespace csa
