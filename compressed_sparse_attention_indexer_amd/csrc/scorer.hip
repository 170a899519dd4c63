// Indexer scorer: s[q, j] = sum_h w[q,h] * act(q_idx[q,h,:] . k_idx_b[j,:]).
// The indexer compares each query against every compressed entry with a
// dot product per indexer head and weights the heads by per-query importance
// weights ("DeepSeek-V4 Architecture Analysis", INNOVATIONS 1, indexer bullet;
// DeepSeek-V4-Flash config: index_n_heads 64, index_head_dim 128).
#include "common.hpp"
#include "launch.hpp"
#include "topk_hist.hpp"
#include "scorer_common.hpp"

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
// registers), B = index keys (dims x entries).  A wave-step of keys is 8 KiB
// of consecutive rows, loaded whole-row (each load instruction reads 1 KiB
// contiguous) with nontemporal loads two steps ahead; to compute, the wave
// copies the step into its own LDS block and reads it back as B fragments
// (lane (e, g) of a tile takes dims [32s + 8g, 32s + 8g + 8) of entry e for
// k-step s), and the registers it freed take the loads of the step two
// ahead before the math starts.  The C tile gives each lane 4 heads of one
// entry; the weighted activation sum over those heads is done in registers
// and the 4 lane groups are summed with two cross-lane adds.
//
// Launch shape: about one 4-wave workgroup per CU.  A workgroup-step covers
// 128 entries (32 KiB of keys); each workgroup takes one contiguous stretch of
// its query's visible steps, and its four waves, lined up by a barrier after
// their first loads, read the four 8 KiB blocks of each step together (on this
// part that streams HBM about 7% faster than dealing the steps round-robin).
// Optionally each workgroup also histograms the keys of the scores it writes,
// for the top-k, and (when the caller asks and its stretch fits in LDS) keeps
// its keys and hands the selection its entries at and above a cut bin.
namespace {
constexpr int kWaveStep = 32;                         // entries per wave and step
constexpr int kWgStep = kBf16WgStep;                  // entries per workgroup step
constexpr int kScoreDepth = 2;                        // key steps in flight per wave
typedef bf16x8_t KeyFrag[2][4];
typedef u32x4_t KeyRaw[8];  // a wave-step of keys as loaded: 8 KiB, 16 B per lane per load
constexpr int kRawRowWords = kDI / 2 + 4;  // LDS row of 128 bf16 + 16 B pad
}  // namespace

template <int kAct, bool kHist, int kDepth>
__global__ __launch_bounds__(64 * kScoreWaves, 1) void index_scores_bf16_kernel(ScoreArgs a) {
    __shared__ uint32_t lh[kHist ? kTopkBins : 1];
    __shared__ uint32_t lkeys[kHist ? kEmitMax : 1];  // keys of this workgroup's stretch (emission)
    __shared__ __attribute__((aligned(16))) uint32_t kraw[kScoreWaves][kWaveStep * kRawRowWords];
    __shared__ int s_red[4];
    __shared__ int s_scan[4];  // the emission's scans (s_red may still be read after the window store)
    __shared__ int s_cut;
    // this workgroup's query, and its part of the query's entries (of n_parts)
    const int qi = blockIdx.y, part = blockIdx.x, n_parts = gridDim.x;
    const int b = qi / a.T;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int e = lane & 15;   // entry (B column) / head row (A row) within a tile
    const int g = lane >> 4;   // dim group within a k-step

    int nvis = visible_entries(a.seq_len[b], a.q_pos[qi], a.ratio);
    nvis = nvis < a.n_max ? nvis : a.n_max;
    const bool with_hist = kHist && nvis > a.K;  // same for the whole workgroup
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
    // Work split: the query's visible entries, in workgroup steps of kWgStep,
    // are cut into n_parts contiguous ranges, one per workgroup, so each
    // workgroup streams one stretch of the key rows; wave w takes entries
    // kWaveStep * w .. + kWaveStep - 1 of each step (step k of this wave starts
    // at entry base0 + k * stride).  Steps wholly past the visible entries get
    // -inf only, dealt round-robin.
    const int vis_steps = (nvis + kWgStep - 1) / kWgStep;
    const int chunk = (vis_steps + n_parts - 1) / n_parts;
    const int s0 = part * chunk;
    const int n_load = vis_steps - s0 < chunk ? (vis_steps - s0 > 0 ? vis_steps - s0 : 0) : chunk;
    const int stride = kWgStep;
    const int base0 = s0 * kWgStep + wave * kWaveStep;
    // emission: the host enables it only when every stretch fits in lkeys (checked
    // here too: a stretch that does not fit marks its region overflowed instead)
    const bool emit = kHist && with_hist && a.em_cap > 0 && n_load * kWgStep <= kEmitMax;
    const int stretch0 = s0 * kWgStep;

    // Every load is unconditional (indices clamped into the visible rows) so
    // the loop body is straight-line code and the compiler can wait for one
    // step's loads while the next step's are still in flight.
    // Loads read whole rows: load i of lane l takes 16 bytes of entry
    // base + 4i + l/16 (1 KiB contiguous per instruction); the step is
    // redistributed into MFMA fragments through a wave-private LDS block.
    auto load = [&](KeyRaw &kr, int base) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int j = base + 4 * i + (lane >> 4);
            j = j < nvis ? j : last;
            kr[i] = __builtin_nontemporal_load(as_global<u32x4_t>(kb + (size_t)j * kDI + 8 * (lane & 15)));
        }
    };
    uint32_t *kw = kraw[wave];
    auto stash = [&](const KeyRaw &kr) {
#pragma unroll
        for (int i = 0; i < 8; ++i) *(u32x4_t *)&kw[(4 * i + (lane >> 4)) * kRawRowWords + 4 * (lane & 15)] = kr[i];
    };
    auto frags = [&](KeyFrag &kf) {
#pragma unroll
        for (int et = 0; et < 2; ++et)
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2)
                kf[et][s2] = *(const bf16x8_t *)&kw[(16 * et + e) * kRawRowWords + 16 * s2 + 4 * g];
    };
    static_assert(kScoreWaves == 4, "the histogram window store takes 256 threads");
    int hmax = -1;  // highest histogram bin this thread added
    // `live`: the step exists (a clamped re-run of the last step stores nothing)
    auto process = [&](KeyRaw &kr, int base, bool live, int next) {
        stash(kr);
        load(kr, next);  // the registers are free again: the next load goes out before this step's math
        KeyFrag kf;
        frags(kf);
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
                    p = fmaf(wr[ht][r], index_act<kAct>(acc[ht][r]), p);
                }
            p = sum_xor16(p);
            p = sum_xor32(p);
            part[et] = p;
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // the fragment reads first
        __builtin_amdgcn_sched_group_barrier(0x008, 32, 0); // then the MFMAs
        // Lanes of group g < 2 store column tile g: 32 consecutive scores.
        const float sv = j < nvis ? (g == 0 ? part[0] : part[1]) : -INFINITY;
        if (live && g < 2 && j < a.n_max) srow[j] = sv;
        if (with_hist) {
            const uint32_t key = order_key(sv);
            const uint32_t bin = key >> 20;
            const bool add = live && g < 2 && j < nvis;
            lds_hist_add(lh, bin, add);
            if (add) hmax = max(hmax, (int)bin);
            if (emit && add) lkeys[j - stretch0] = key;
        }
    };

    // Software pipeline kDepth steps deep, unrolled by kDepth so that no load
    // sits behind a branch: while step k computes, the loads of steps k+1 ..
    // k+kDepth-1 are in flight.  Steps past the last one reload the last step
    // and store nothing.  The histogram is cleared while the first loads are
    // out; then the waves meet at a barrier (every wave reaches it, with or
    // without steps), so the four go on loading adjacent 8 KiB blocks of their
    // workgroup's stretch together rather than drifting apart from their
    // staggered starts (measured: 47.0 -> 43.7 us for batch 4 x 262,144
    // entries, against 46.4 us with the barrier and round-robin steps).
    KeyRaw kbuf[kDepth];
    auto step = [&](int k) { return base0 + (k < n_load ? k : n_load - 1) * stride; };
    if (n_load > 0) {
#pragma unroll
        for (int i = 0; i < kDepth; ++i) load(kbuf[i], step(i));
    }
    if (with_hist) {
        for (int i = threadIdx.x; i < kTopkBins; i += 64 * kScoreWaves) lh[i] = 0u;
    }
    __syncthreads();
    if (n_load > 0) {
        for (int k = 0; k < n_load; k += kDepth) {
#pragma unroll
            for (int i = 0; i < kDepth; ++i) {
                process(kbuf[i], step(k + i), k + i < n_load, step(k + i + kDepth));
            }
        }
    }
    const int all_steps = (a.n_max + kWgStep - 1) / kWgStep;
    for (int st = vis_steps + part; st < all_steps; st += n_parts) {  // steps past the visible entries
        const int j = st * kWgStep + wave * kWaveStep + 16 * g + e;
        if (g < 2 && j < a.n_max) srow[j] = -INFINITY;
    }
    if (with_hist) {
        const size_t w = (size_t)qi * n_parts + part;
        const int top = hist_window_store_top(lh, hmax, a.win_hdr + w, a.win_cnt + w * kTopkWin, s_red);
        decode_emission<64 * kScoreWaves>(a, lh, lkeys, emit, nvis, s0, n_load, kWgStep, w, top, s_scan, &s_cut);
    }
}

// ---------------------------------------------------------------------------
// bf16 MFMA scorer for many queries of one sequence (prefill chunk), HI = 64,
// DI = 128.  Here the work is a dense contraction [queries*64 x 128] x
// [128 x entries] with a per-(query, entry) epilogue, so it is tiled like a
// GEMM: a workgroup of 8 waves takes 8 consecutive queries of one sequence
// (one per wave, its 64 x 128 index matrix resident in registers as A
// fragments) and a chunk of entries, which streams through LDS 128 entries at
// a time (double-buffered, the next tile's global loads in flight while the
// current one is computed).  Each B fragment read from LDS feeds 4 MFMAs (the
// 4 head tiles).  Per 16-entry column tile, a lane holds 16 heads of one
// entry; it folds them with the weights and activation in registers, and a
// 3-exchange butterfly over the 4 lane groups leaves lane l with the score of
// entry l of each 64-entry group, stored as one coalesced 256-byte row
// segment.  The per-element epilogue (activation + weighted add: two VALU
// instructions per 256 MFMA flops) runs beside the other wave's MFMAs.
//
// Selection in the fused call (kMode): none (the scores alone), histogram
// windows (each wave keeps its query's key histogram over the chunk beside
// the scores it writes; the top-k then emits and selects from the scores), or
// streaming: no score is written; each wave keeps its query's K best entries
// of the chunk in LDS (see wave_keep_top) and writes them as the chunk's
// region for the selection, which then never reads a score row.
//
// Workgroup order: when the entry chunks come in multiples of 8, the
// workgroups sharing an entry chunk are dealt to one XCD (hardware deals
// consecutive workgroup ids round-robin over the 8 XCDs), so the key tiles
// they stream are shared through that XCD's L2.
namespace {
constexpr int kPfWaves = 8;                  // two waves per SIMD
constexpr int kPfQW = 1;                     // queries per wave
constexpr int kPfQueries = kPfQW * kPfWaves; // queries per workgroup
constexpr int kPfTile = 128;                 // entries per LDS tile
constexpr int kPfRowWords = kDI / 2 + 4;     // LDS row: 128 bf16 + 16 B pad (conflict-free reads)
constexpr int kPfTileWords = kPfTile * kPfRowWords;
constexpr int kPfTargetWgs = 2048;           // about 8 workgroups per CU over the launch
constexpr int kPfStage = kPfTile * (kDI / 8) / (64 * kPfWaves);  // 16-byte tile chunks per thread
static_assert(kPfStage * 64 * kPfWaves == kPfTile * (kDI / 8), "tile staging covers the tile");
static_assert(kPfTile % 64 == 0, "whole 64-entry groups per tile");
constexpr int kSelNone = 0, kSelHist = 1, kSelStream = 2;  // the tiled kernel's selection modes
constexpr int kSelBuf = 1920;                  // stream buffer per wave (entries: key + 16-bit chunk offset)
constexpr int kSelSlots = kSelBuf / 64;        // buffer entries per lane
constexpr int kSelSlack = 256;                 // a compaction inside the chunk keeps K .. K + kSelSlack entries
static_assert(kSelBuf % 64 == 0, "whole lanes per buffer");
static_assert(kSelKeepMax + kSelSlack + kPfTile <= kSelBuf - kPfTile, "a compaction leaves room for a tile");
}  // namespace

// Stream selection, one wave: of the n entries in its LDS buffer (keys bk,
// chunk offsets bo, in index order; n > K), keep the best ones in place and
// in index order, set n to their count and return a key t such that the chunk's
// K best so far are all kept and every entry met later (a higher index) needs
// a key above t to be among them.  The keys are held in registers; t is found
// bit by bit from the top (the largest value with at least K keys at or above
// it), starting below the bits all the keys share.  exact: t is the K-th key,
// and exactly K entries are kept (every key above t and the first ones equal
// to it: equal keys rank by lower index).  Otherwise the search stops as soon
// as no more than K + kSelSlack keys are at or above t, and all of them are
// kept (then at least K keys are at or above t, so a later entry with key t
// or below ranks under K of them).  LDS accesses of one wave complete in
// issue order, so the in-place writes (each to a slot at or below the one it
// came from, after the reads of its 64-slot group) need no barrier.
__device__ __forceinline__ uint32_t wave_keep_top(uint32_t *bk, uint16_t *bo, int &n, int K, bool exact) {
    const int lane = threadIdx.x & 63;
    const uint64_t lt = lanemask_lt();
    uint32_t k[kSelSlots];
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int s = 0; s < kSelSlots; ++s) {
        const bool live = 64 * s + lane < n;
        k[s] = live ? bk[64 * s + lane] : 0u;  // live keys are > 0
        kmin = live ? min(kmin, k[s]) : kmin;
        kmax = max(kmax, k[s]);
    }
    // unsigned wave maximum through the signed one (bias by 2^31); the minimum as ~max(~x)
    auto umax = [](uint32_t x) { return (uint32_t)wave_max_int((int)(x ^ 0x80000000u)) ^ 0x80000000u; };
    kmin = ~umax(~kmin);
    kmax = umax(kmax);
    // every live key shares kmax's bits above the highest bit where kmin and kmax differ
    const uint32_t diff = kmin ^ kmax;
    const int top = diff ? 31 - __builtin_clz(diff) : -1;
    uint32_t t = diff == 0u ? kmax : (top == 31 ? 0u : kmax & ~((2u << top) - 1u));
    int cnt_t = n;  // keys at or above t
#pragma unroll 1
    for (int b = top; b >= 0; --b) {
        if (!exact && cnt_t <= K + kSelSlack) break;
        const uint32_t c = t | (1u << b);
        int cnt = 0;
#pragma unroll
        for (int s = 0; s < kSelSlots; ++s) cnt += k[s] >= c;
        cnt = __builtin_amdgcn_readlane(wave_incl_scan(cnt), 63);
        if (cnt >= K) {
            t = c;
            cnt_t = cnt;
        }
    }
    // equal keys that stop the search short of K + kSelSlack: keep exactly K
    if (cnt_t > K + kSelSlack) exact = true;
    int n_eq = n;  // keys equal to t kept: all of them unless exact
    if (exact) {
        int above = 0;
#pragma unroll
        for (int s = 0; s < kSelSlots; ++s) above += k[s] > t;
        n_eq = K - __builtin_amdgcn_readlane(wave_incl_scan(above), 63);
    }
    int w = 0, eq_seen = 0;
#pragma unroll
    for (int s = 0; s < kSelSlots; ++s) {
        const bool eq = k[s] == t;
        const uint64_t em = __ballot(eq);
        const bool keep = k[s] > t || (eq && eq_seen + __popcll(em & lt) < n_eq);
        const uint64_t km = __ballot(keep);
        if (keep) {
            const int p = w + __popcll(km & lt);
            const uint16_t o = bo[64 * s + lane];
            bk[p] = k[s];
            bo[p] = o;
        }
        w += __popcll(km);
        eq_seen += __popcll(em);
    }
    n = w;
    return t;
}

struct TiledPlan {
    int qb_per_seq;        // query blocks per sequence
    int n_chunks;          // entry chunks
    int tiles_per_chunk;
};

static TiledPlan tiled_plan(const ScoreArgs &a) {
    TiledPlan p;
    p.qb_per_seq = (a.T + kPfQueries - 1) / kPfQueries;
    const int n_qb = a.B * p.qb_per_seq;
    const int n_tiles = (a.n_max + kPfTile - 1) / kPfTile;
    int want = (kPfTargetWgs + n_qb - 1) / n_qb;
    if (want >= 8) want = (want + 7) / 8 * 8;
    if (want > n_tiles) want = n_tiles;
    if (want < 1) want = 1;
    p.tiles_per_chunk = (n_tiles + want - 1) / want;
    p.n_chunks = (n_tiles + p.tiles_per_chunk - 1) / p.tiles_per_chunk;
    return p;
}

template <int kAct, int kMode>
__global__ __launch_bounds__(64 * kPfWaves, 1) void index_scores_tiled_kernel(ScoreArgs a, TiledPlan pl) {
    constexpr bool kHist = kMode == kSelHist, kStream = kMode == kSelStream;
    static_assert((!kHist && !kStream) || kPfQW == 1, "one histogram or selection per wave holds one query");
    __shared__ __attribute__((aligned(16))) uint32_t kt[2][kPfTileWords];
    __shared__ int s_nv[kPfWaves];
    // Optional top-k key-histogram window of each wave's query over this
    // workgroup's chunk.  Only the kTopkWin bins at and below the highest bin
    // seen so far (m_top, the same in every lane) are kept, as lane-private
    // counters: bin m_top - o of lane l is word 64 * o + l, so the 64 lanes of
    // an add touch 64 different banks and never wait on one another.  A score
    // above m_top is held back in a register until the end of its tile; then
    // every lane shifts its counters down by the rise and adds what it held.
    // The 64-entry groups themselves stay free of branches.
    __shared__ uint32_t lh[kHist ? kPfWaves : 1][kHist ? kTopkWin * 64 : 1];
    int m_top = -1;
    // Stream selection: each wave's buffer of entries (key, offset in the
    // chunk) above its threshold sel_thr, sel_n of them, in index order
    // (sel_n and sel_thr are the same in every lane of the wave).  A wave whose
    // buffer could overflow in the next tile raises its flag at the end of a
    // tile; after the next tile's barrier every wave sees the flags, and if
    // any is up, every wave holding more than K + kSelSlack entries compacts
    // then, so the workgroup waits at its barriers for one round of
    // compactions instead of one per wave.
    __shared__ uint32_t sel_key[kStream ? kPfWaves : 1][kStream ? kSelBuf : 1];
    __shared__ uint16_t sel_off[kStream ? kPfWaves : 1][kStream ? kSelBuf : 1];
    __shared__ int sel_flag[kStream ? 2 : 1][kPfWaves];  // by tile parity
    int sel_n = 0;
    uint32_t sel_thr = 0u;  // live keys are > 0
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int e = lane & 15, g = lane >> 4;

    // workgroup -> (query block, entry chunk)
    const int n_qb = a.B * pl.qb_per_seq;
    int qb, ec;
    if (pl.n_chunks % 8 == 0) {
        const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
        qb = slot % n_qb;
        ec = (slot / n_qb) * 8 + xcd;
    } else {
        qb = blockIdx.x % n_qb;
        ec = blockIdx.x / n_qb;
    }
    const int b = qb / pl.qb_per_seq;
    const int t0 = (qb % pl.qb_per_seq) * kPfQueries + kPfQW * wave;
    const int64_t L = a.seq_len[b];

    // this wave's queries (a query past T repeats the last one and stores nothing)
    int qi[kPfQW], nv[kPfQW];
    bool qok[kPfQW];
    int nv_wave = 0;
#pragma unroll
    for (int q = 0; q < kPfQW; ++q) {
        const int t = t0 + q;
        qok[q] = t < a.T;
        qi[q] = b * a.T + (qok[q] ? t : a.T - 1);
        const int v = visible_entries(L, a.q_pos[qi[q]], a.ratio);
        nv[q] = v < a.n_max ? v : a.n_max;
        if (qok[q]) nv_wave = max(nv_wave, nv[q]);
    }
    if (lane == 0) s_nv[wave] = nv_wave;

    bf16x8_t qa[kPfQW][4][4];
    float wr[kPfQW][4][4];
#pragma unroll
    for (int q = 0; q < kPfQW; ++q) {
        const uint16_t *qsrc = (const uint16_t *)a.q_idx + (size_t)qi[q] * kHI * kDI;
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
                qa[q][ht][s] = *(const bf16x8_t *)(qsrc + (16 * ht + e) * kDI + 32 * s + 8 * g);
#pragma unroll
            for (int r = 0; r < 4; ++r) wr[q][ht][r] = a.w[(size_t)qi[q] * kHI + 16 * ht + 4 * g + r];
        }
    }
    const bool with_hist = kHist && qok[0] && nv[0] > a.K;  // one query per wave: its own histogram
    const bool with_sel = kStream && qok[0] && nv[0] > a.K;
    if (kHist) {
        for (int i = tid; i < kPfWaves * kTopkWin * 64; i += 64 * kPfWaves) (&lh[0][0])[i] = 0u;
    }
    if (kStream && tid < 2 * kPfWaves) (&sel_flag[0][0])[tid] = 0;
    __syncthreads();
    int nv_max = 0;
#pragma unroll
    for (int w = 0; w < kPfWaves; ++w) nv_max = max(nv_max, s_nv[w]);

    const int j0 = ec * pl.tiles_per_chunk * kPfTile;
    const int j_end = min(j0 + pl.tiles_per_chunk * kPfTile, a.n_max);
    // tiles holding an entry some query of the block sees
    const int n_ct = nv_max > j0 ? (min(j_end, nv_max) - j0 + kPfTile - 1) / kPfTile : 0;
    const uint16_t *kb = (const uint16_t *)a.k_idx[b];
    const int last = nv_max > 0 ? nv_max - 1 : 0;

    // staging: thread -> kPfStage chunks of 16 bytes (entry c/16, dims 8*(c%16) .. +8)
    u32x4_t st[kPfStage];
    auto fetch = [&](int tile) {
#pragma unroll
        for (int u = 0; u < kPfStage; ++u) {
            const int c = tid + 64 * kPfWaves * u;
            int j = j0 + tile * kPfTile + (c >> 4);
            j = j < nv_max ? j : last;
            st[u] = *as_global<u32x4_t>(kb + (size_t)j * kDI + 8 * (c & 15));
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int u = 0; u < kPfStage; ++u) {
            const int c = tid + 64 * kPfWaves * u;
            *(u32x4_t *)&kt[buf][(c >> 4) * kPfRowWords + 4 * (c & 15)] = st[u];
        }
    };

    if (n_ct > 0) fetch(0);
    for (int tile = 0; tile < n_ct; ++tile) {
        const int buf = tile & 1;
        stash(buf);
        if (tile + 1 < n_ct) fetch(tile + 1);
        __syncthreads();
        if (kStream) {  // a round of compactions when some wave's buffer could overflow in this tile
            int any = 0;
#pragma unroll
            for (int w2 = 0; w2 < kPfWaves; ++w2) any |= sel_flag[tile & 1][w2];
            if (any && sel_n > a.K + kSelSlack)
                sel_thr = wave_keep_top(sel_key[wave], sel_off[wave], sel_n, a.K, false);
        }
        int held[kPfTile / 64];  // per group: a bin above m_top, else -1
#pragma unroll
        for (int grp = 0; grp < kPfTile / 64; ++grp) {  // 64 entries: one butterfly and store
            float p[kPfQW][4];
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                bf16x8_t kf[4];
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    kf[s] = *(const bf16x8_t *)&kt[buf][(64 * grp + 16 * sb + e) * kPfRowWords + 16 * s + 4 * g];
#pragma unroll
                for (int q = 0; q < kPfQW; ++q) {
                    f32x4_t acc[4];
#pragma unroll
                    for (int ht = 0; ht < 4; ++ht) {
                        acc[ht] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int s = 0; s < 4; ++s)
                            acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[q][ht][s], kf[s], acc[ht], 0, 0, 0);
                    }
                    float x = 0.f;
#pragma unroll
                    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
                        for (int r = 0; r < 4; ++r) x = fmaf(wr[q][ht][r], index_act<kAct>(acc[ht][r]), x);
                    p[q][sb] = x;  // entry 16*sb + e, heads of lane group g
                }
            }
            // butterfly over the lane groups: lane 16g + e ends with entry 16g + e summed over all heads
            const int j = j0 + tile * kPfTile + 64 * grp + lane;
#pragma unroll
            for (int q = 0; q < kPfQW; ++q) {
                float k2[2];
#pragma unroll
                for (int k = 0; k < 2; ++k) {  // lower half keeps p[k], upper half p[2 + k]
                    const LanePair pr = pair32(p[q][k], p[q][2 + k]);
                    k2[k] = pr.lo + pr.hi;
                }
                const LanePair pr = pair16(k2[0], k2[1]);  // lane group lo keeps k2[lo]
                const float tot = pr.lo + pr.hi;
                if (!kStream && qok[q] && j < a.n_max)
                    a.scores[(size_t)qi[q] * a.n_max + j] = j < nv[q] ? tot : -INFINITY;
                if (kStream) {
                    const uint32_t key = order_key(tot);
                    const bool take = with_sel && j < nv[q] && key > sel_thr;
                    const uint64_t m = __ballot(take);
                    if (m) {
                        if (take) {
                            const int p = sel_n + __popcll(m & lanemask_lt());
                            sel_key[wave][p] = key;
                            sel_off[wave][p] = (uint16_t)(j - j0);
                        }
                        sel_n += __popcll(m);
                    }
                }
                if (kHist) {
                    const bool v = with_hist && j < nv[q];
                    const int bin = (int)(order_key(tot) >> 20);
                    const bool up = v && bin > m_top;
                    held[grp] = up ? bin : -1;
                    const int o = m_top - bin;
                    const bool in = v && !up && o < kTopkWin;
                    atomicAdd(&lh[wave][64 * (in ? o : 0) + lane], in ? 1u : 0u);
                }
            }
        }
        if (kHist) {
            int hm = held[0];
#pragma unroll
            for (int g2 = 1; g2 < kPfTile / 64; ++g2) hm = max(hm, held[g2]);
            if (__ballot(hm > m_top)) {  // the top bin rose in this tile (rare after the first)
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) hm = max(hm, __shfl_xor(hm, o));
                const int d = hm - m_top;
                uint32_t *hw = &lh[wave][lane];
#pragma unroll
                for (int o = kTopkWin - 1; o >= 0; --o) hw[64 * o] = o >= d ? hw[64 * (o - d)] : 0u;
                m_top = hm;
#pragma unroll
                for (int g2 = 0; g2 < kPfTile / 64; ++g2)
                    if (held[g2] >= 0 && m_top - held[g2] < kTopkWin) hw[64 * (m_top - held[g2])] += 1u;
            }
        }
        // the flag for the next tile (read after its barrier)
        if (kStream && lane == 0) sel_flag[(tile + 1) & 1][wave] = sel_n > kSelBuf - kPfTile;
    }
    // entries of the chunk no query of the block sees
    if (!kStream)
        for (int jj = j0 + n_ct * kPfTile + lane; jj < j_end; jj += 64)
#pragma unroll
            for (int q = 0; q < kPfQW; ++q)
                if (qok[q]) a.scores[(size_t)qi[q] * a.n_max + jj] = -INFINITY;
    if (with_sel) {
        // the chunk's region: its best K entries in index order, the slots past
        // them key 0 (no live key is 0); header {cut 0, count}
        if (sel_n > a.K) wave_keep_top(sel_key[wave], sel_off[wave], sel_n, a.K, true);
        const size_t w = (size_t)qi[0] * pl.n_chunks + ec;
        uint32_t *okey = a.em_key + w * a.em_cap;
        int32_t *oidx = a.em_idx + w * a.em_cap;
        for (int i = lane; i < a.em_cap; i += 64) {
            const bool live = i < sel_n;
            okey[i] = live ? sel_key[wave][i] : 0u;
            if (live) oidx[i] = j0 + sel_off[wave][i];
        }
        if (lane == 0) {
            a.em_hdr[2 * w] = 0;
            a.em_hdr[2 * w + 1] = sel_n;
        }
    }
    if (kHist) __syncthreads();  // the wave's histogram atomics are done before it is read
    if (with_hist) {
        // the chunk's window as the top-k expects it: hdr = highest non-empty bin
        // M (-1 if none), cnt[t] = count of bin M - (kTopkWin - 1) + t.  Lane t
        // sums counter kTopkWin - 1 - t over all lanes, starting at its own
        // lane so that the 32 reads of a step fall into 32 banks.
        const size_t w = (size_t)qi[0] * pl.n_chunks + ec;
        if (lane < kTopkWin) {
            const uint32_t *row = &lh[wave][64 * (kTopkWin - 1 - lane)];
            uint32_t c = 0;
#pragma unroll 16
            for (int k = 0; k < 64; ++k) c += row[(k + lane) & 63];
            a.win_cnt[w * kTopkWin + lane] = m_top - (kTopkWin - 1) + lane >= 0 ? c : 0u;
        }
        if (lane == 0) a.win_hdr[w] = m_top;
    }
}

bool score_uses_tiles(int dtype, int T) { return dtype == kBF16 && T >= kPfQueries; }

hipError_t launch_index_scores(const ScoreArgs &a, int dtype, hipStream_t stream) {
    const int Q = a.B * a.T;
    if (dtype == kF32) {
        dim3 grid((a.n_max + 255) / 256, Q);
        const size_t lds = sizeof(float) * (size_t)(a.HI * a.DI + a.HI);
        hipLaunchKernelGGL(index_scores_f32_kernel, grid, dim3(256), lds, stream, a);
        return hipGetLastError();
    }
    if (score_uses_tiles(dtype, a.T)) {
        const TiledPlan pl = tiled_plan(a);
        const dim3 grid(a.B * pl.qb_per_seq * pl.n_chunks), block(64 * kPfWaves);
        // the caller sized the windows (or the stream regions) with tiled_windows
        const int mode = a.sel_stream ? kSelStream : (a.win_hdr != nullptr ? kSelHist : kSelNone);
        if (mode == kSelStream &&
            (a.K < 1 || a.K > kSelKeepMax || a.em_cap < a.K || pl.tiles_per_chunk * kPfTile > kSelChunkMax))
            return hipErrorInvalidValue;
        if (a.act == 0) {
            if (mode == kSelStream)
                hipLaunchKernelGGL((index_scores_tiled_kernel<0, kSelStream>), grid, block, 0, stream, a, pl);
            else if (mode == kSelHist)
                hipLaunchKernelGGL((index_scores_tiled_kernel<0, kSelHist>), grid, block, 0, stream, a, pl);
            else
                hipLaunchKernelGGL((index_scores_tiled_kernel<0, kSelNone>), grid, block, 0, stream, a, pl);
        } else {
            if (mode == kSelStream)
                hipLaunchKernelGGL((index_scores_tiled_kernel<1, kSelStream>), grid, block, 0, stream, a, pl);
            else if (mode == kSelHist)
                hipLaunchKernelGGL((index_scores_tiled_kernel<1, kSelHist>), grid, block, 0, stream, a, pl);
            else
                hipLaunchKernelGGL((index_scores_tiled_kernel<1, kSelNone>), grid, block, 0, stream, a, pl);
        }
        return hipGetLastError();
    }
    const dim3 grid(score_workgroups(a.n_max, Q), Q);
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

int tiled_windows(int B, int T, int n_max) {
    ScoreArgs a{};
    a.B = B;
    a.T = T;
    a.n_max = n_max;
    return tiled_plan(a).n_chunks;
}

int tiled_chunk_entries(int B, int T, int n_max) {
    ScoreArgs a{};
    a.B = B;
    a.T = T;
    a.n_max = n_max;
    return tiled_plan(a).tiles_per_chunk * kPfTile;
}

int tiled_emit_cap(int B, int T, int n_max, int K) {
    const int n = tiled_windows(B, T, n_max);
    const int cap = decode_region_cap(n, K, tiled_chunk_entries(B, T, n_max));
    // room for the streaming selection's regions (a chunk's K best) when the
    // selection can hold them all
    const int ks = (K + 15) / 16 * 16;
    if (K <= kSelKeepMax && (long)n * ks <= kTopkMaxSlots) return cap > ks ? cap : ks;
    return cap;
}

int score_workgroups(int n_max, int n_queries) { return decode_score_workgroups(n_max, n_queries, kWgStep); }

DecodeGeom decode_geom(bool fp8, int n_max, int n_queries, int K) {
    return decode_geom_for(n_max, n_queries, K, fp8 ? kFp8WgStep : kBf16WgStep);
}

}  // namespace csa
