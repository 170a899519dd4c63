// Per-query top-k over the indexer scores (DeepSeek-V4-Flash config:
// index_topk 512; "DeepSeek-V4 Architecture Analysis", INNOVATIONS 1, indexer
// bullet).  Order is (fp32 score desc, index asc); the K chosen indices are
// written ascending, padded with -1 when fewer than K entries are visible.
//
// Scores become order-preserving uint32 keys.  Three row-length regimes:
//  * up to kTopkSmallMax entries: one 1024-thread workgroup per query keeps
//    the row in LDS, finds the exact K-th key with four 8-bit radix passes and
//    writes the selection in index order with an ordered compaction.
//  * up to kTopkOneKernelMax: the key histogram comes in windows (one per
//    scorer or histogram workgroup, plain stores); one workgroup per query
//    merges them into the exact histogram of the top kTopkWin bins (1/8
//    octave each, just below the largest key), finds the bin holding the K-th
//    key, scans the row into "above" and "candidate" lists in LDS (ordered
//    compaction, so both are in index order), selects among the candidates
//    and merges the two lists into the ascending output.
//  * longer rows: many workgroups each merge the windows into the threshold
//    and scan a slice of the row, writing their own lists with plain stores;
//    one workgroup per query then gathers the lists and selects.
// Every shortcut is checked (counts consistent, buffers not overflowed,
// threshold inside the merged window); otherwise the exact whole-row radix
// scan runs.  No step uses global atomics, and correctness never depends on
// the workspace's prior contents.
#include "common.hpp"
#include "launch.hpp"
#include "topk_hist.hpp"

namespace csa {

namespace {
constexpr int kWG = 1024;
constexpr int kWaves = kWG / 64;
constexpr int kAuxThreads = 256;
constexpr int kPerThread = kTopkAuxChunk / kAuxThreads;  // 8 scores per thread
constexpr int kSubCap = 1024;                            // candidates sharing the final sub-bin
constexpr int kFinalGroup = 8;                           // selection: threads per filter region
constexpr int kSpecC = 2;                                // candidates per thread loaded in the first round


// Shared state of the radix selection for a workgroup of NT threads.
template <int NT>
struct TopkSharedT {
    uint32_t hist[256];
    uint64_t masks[2][NT / 64][2];
    int bcast[4];
};
using TopkShared = TopkSharedT<kWG>;

// Wave 0 finds the histogram bin that holds the need-th largest element
// (counting from bin 255 down) and publishes (bin, rank within the bin).
template <int NT>
__device__ __forceinline__ void find_bin_256(TopkSharedT<NT> &sh, int need) {
    const int lane = threadIdx.x & 63;
    if (threadIdx.x < 64) {
        uint32_t h[4];
        uint32_t s = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            h[i] = sh.hist[4 * lane + i];
            s += h[i];
        }
        const uint32_t inc = wave_incl_scan_u(s);
        const uint32_t suf = __builtin_amdgcn_readlane(inc, 63) - inc + s;  // sum over lanes >= this lane
        const uint32_t above = suf - s;
        if (above < (uint32_t)need && (uint32_t)need <= suf) {
            uint32_t a = above;
            for (int i = 3; i >= 0; --i) {
                if (a < (uint32_t)need && (uint32_t)need <= a + h[i]) {
                    sh.bcast[0] = 4 * lane + i;
                    sh.bcast[1] = need - (int)a;
                    break;
                }
                a += h[i];
            }
        }
    }
}

// Exact top-k of one row (n visible entries) by one workgroup of NT threads.
template <bool kInLds, int NT = kWG>
__device__ void topk_row(const float *__restrict__ row, int n, int K, int32_t *__restrict__ out,
                         uint32_t *keys, TopkSharedT<NT> &sh) {
    constexpr int kWG = NT, kWaves = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (n <= K) {
        for (int i = tid; i < K; i += kWG) out[i] = i < n ? i : -1;
        return;
    }
    if (kInLds) {
        for (int i = tid; i < n; i += kWG) keys[i] = order_key(row[i]);
        __syncthreads();
    }
    auto key_at = [&](int i) -> uint32_t { return kInLds ? keys[i] : order_key(row[i]); };

    // 1. Exact K-th largest key: four 8-bit digits from the top.
    uint32_t prefix = 0;
    int need = K;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
        if (tid < 256) sh.hist[tid] = 0;
        __syncthreads();
        for (int i0 = 0; i0 < n; i0 += kWG) {
            const int i = i0 + tid;
            const uint32_t k = i < n ? key_at(i) : 0u;
            lds_hist_add(sh.hist, (k >> shift) & 255u, i < n && (k & hi_mask) == prefix);
        }
        __syncthreads();
        find_bin_256(sh, need);
        __syncthreads();
        prefix |= (uint32_t)sh.bcast[0] << shift;
        need = sh.bcast[1];
        __syncthreads();
    }
    const uint32_t T = prefix;  // K-th largest key; `need` of the keys equal to T are taken

    // 2. Ordered compaction: keys > T, and the first `need` keys == T by index.
    int base_eq = 0, base_sel = 0, buf = 0;
    const uint64_t lt = lanemask_lt();
    for (int r0 = 0; r0 < n; r0 += kWG) {
        const int i = r0 + tid;
        const uint32_t k = i < n ? key_at(i) : 0u;
        const bool gt = i < n && k > T;
        const bool eq = i < n && k == T;
        const uint64_t mg = __ballot(gt), me = __ballot(eq);
        if (lane == 0) {
            sh.masks[buf][wave][0] = mg;
            sh.masks[buf][wave][1] = me;
        }
        __syncthreads();
        int eq_before = base_eq, sel_before = base_sel;
        int my_sel_before = 0, my_take = 0;
        for (int w = 0; w < kWaves; ++w) {
            const uint64_t g2 = sh.masks[buf][w][0], e2 = sh.masks[buf][w][1];
            const int ce = __popcll(e2);
            int take = need - eq_before;
            take = take < 0 ? 0 : (take > ce ? ce : take);
            if (w == wave) {
                my_sel_before = sel_before;
                my_take = take;
            }
            eq_before += ce;
            sel_before += __popcll(g2) + take;
        }
        const int eq_rank = __popcll(me & lt);
        if (gt || (eq && eq_rank < my_take)) {
            const int pos = my_sel_before + __popcll(mg & lt) + (eq_rank < my_take ? eq_rank : my_take);
            out[pos] = i;
        }
        base_eq = eq_before;
        base_sel = sel_before;
        buf ^= 1;
        if (base_sel >= K) break;  // identical in every thread
    }
}

__device__ __forceinline__ int query_visible(const TopkArgs &a, int qi) {
    const int b = qi / a.T;
    const int n = visible_entries(a.seq_len[b], a.q_pos[qi], a.ratio);
    return n < a.n_max ? n : a.n_max;
}

// R consecutive scores j_first .. j_first + R - 1 of a row (0 past n).  Whole
// 16-byte loads when the chunk lies inside the row and the row is aligned.
template <int R>
__device__ __forceinline__ void load_chunk(const float *row, int j_first, int n, int n_max, bool vec, float (&x)[R]) {
    if (vec && j_first + R <= n_max) {
#pragma unroll
        for (int k = 0; k < R; k += 4) {
            const float4 f = *(const float4 *)(row + j_first + k);
            x[k] = f.x;
            x[k + 1] = f.y;
            x[k + 2] = f.z;
            x[k + 3] = f.w;
        }
#pragma unroll
        for (int k = 0; k < R; ++k)
            if (j_first + k >= n) x[k] = 0.f;
    } else {
#pragma unroll
        for (int k = 0; k < R; ++k) x[k] = j_first + k < n ? row[j_first + k] : 0.f;
    }
}

// Ordered compaction of one round: thread t owns the R consecutive entries
// starting at j_first (the threads' chunks consecutive in thread order).
// Entries whose key bin is above `bin` go to v, those in `bin` to
// (c_key, c_idx), both in index order after the n_gt / n_eq already there;
// writes past a capacity are dropped (the counts still grow, so the caller
// sees the overflow).  n_gt and n_eq are the same in every thread.
template <int NT, int R>
__device__ __forceinline__ void classify_ordered(const float (&x)[R], int j_first, int n, uint32_t bin, int *s_wave,
                                                 int &n_gt, int &n_eq, int32_t *v, int v_cap, uint32_t *c_key,
                                                 int32_t *c_idx, int c_cap) {
    int g = 0, q = 0;
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const uint32_t d = order_key(x[k]) >> 20;
        const bool ok = j_first + k < n;
        g += ok && d > bin;
        q += ok && d == bin;
    }
    int tot;
    const int pre = block_scan_excl<NT>(g | (q << 16), s_wave, &tot);  // per-field sums stay below 2^16
    int sg = n_gt + (pre & 0xFFFF), sq = n_eq + (pre >> 16);
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int j = j_first + k;
        const uint32_t key = order_key(x[k]);
        const uint32_t d = key >> 20;
        if (j < n && d > bin) {
            if (sg < v_cap) v[sg] = j;
            ++sg;
        }
        if (j < n && d == bin) {
            if (sq < c_cap) {
                c_key[sq] = key;
                c_idx[sq] = j;
            }
            ++sq;
        }
    }
    n_gt += tot & 0xFFFF;
    n_eq += tot >> 16;
}

template <int NT>
struct SelectSharedT {
    uint32_t words[256];               // second-level histogram
    int32_t sel[kTopkMaxK];            // chosen candidates in index order (ordered selection)
    uint32_t sub_key[kSubCap];
    int32_t sub_idx[kSubCap];
    int s_wave[NT / 64];
    int cnt[2];
    int bcast[2];
};
using SelectShared = SelectSharedT<kWG>;

// Ordered selection: v[0..na) (entries above the threshold bin) and the
// candidates c_key/c_idx[0..nc) (inside it) are both in index order, na < K,
// na + nc >= K, nc <= kTopkCand.  Thread t takes the consecutive candidates
// [C t, C t + C), C = ceil(nc / kWG).  A candidate is chosen if its
// second-level bin (key bits 19..12) lies above the bin b2 that holds the
// need-th best candidate, or inside b2 with fewer than need2 better
// candidates there ((key, lower index) order; b2's members are gathered in
// LDS first).  The chosen ones are compacted in index order and merged with v
// into `out` by binary search.  Returns false (nothing written, same in every
// thread) if b2 holds more than kSubCap candidates.
template <int NT = kWG>
__device__ bool select_ordered(const int32_t *v, int na, const uint32_t *c_key, const int32_t *c_idx, int nc, int K,
                               int32_t *out, SelectSharedT<NT> &ss) {
    constexpr int kWG = NT;
    constexpr int kMaxC = kTopkCand / kWG;
    const int tid = threadIdx.x;
    const int need = K - na;
    const int C = (nc + kWG - 1) / kWG;
    const int i0 = C * tid;
    uint32_t *h = ss.words;
    if (tid < 256) h[tid] = 0u;
    if (tid == 0) ss.cnt[0] = 0;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kMaxC; ++c)
        if (c < C && i0 + c < nc) atomicAdd(&h[(c_key[i0 + c] >> 12) & 0xFFu], 1u);
    __syncthreads();
    if (tid < 64) {  // wave 0: bins from the top, 4 per lane
        uint32_t cb[4], sum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            cb[i] = h[255 - (4 * tid + i)];
            sum += cb[i];
        }
        const uint32_t incl = wave_incl_scan_u(sum);  // inclusive prefix over lanes (lane 0 = top bins)
        uint32_t acc = incl - sum;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (acc < (uint32_t)need && (uint32_t)need <= acc + cb[i]) {
                ss.bcast[0] = 255 - (4 * tid + i);
                ss.bcast[1] = need - (int)acc;
            }
            acc += cb[i];
        }
    }
    __syncthreads();
    const uint32_t b2 = (uint32_t)ss.bcast[0];
    const int need2 = ss.bcast[1];
#pragma unroll
    for (int c = 0; c < kMaxC; ++c) {  // gather b2's members (any order)
        if (c < C && i0 + c < nc && ((c_key[i0 + c] >> 12) & 0xFFu) == b2) {
            const int slot = atomicAdd(&ss.cnt[0], 1);
            if (slot < kSubCap) {
                ss.sub_key[slot] = c_key[i0 + c];
                ss.sub_idx[slot] = c_idx[i0 + c];
            }
        }
    }
    __syncthreads();
    const int m2 = ss.cnt[0];
    if (m2 > kSubCap) return false;
    uint32_t takes = 0;  // bit c: candidate i0 + c is chosen
#pragma unroll
    for (int c = 0; c < kMaxC; ++c) {
        if (!(c < C && i0 + c < nc)) continue;
        const uint32_t key = c_key[i0 + c];
        const uint32_t bk = (key >> 12) & 0xFFu;
        bool take = bk > b2;
        if (bk == b2) {
            const uint64_t mine = ((uint64_t)key << 32) | (uint32_t)~(uint32_t)c_idx[i0 + c];
            int better = 0;
            for (int u = 0; u < m2; ++u)
                better += (((uint64_t)ss.sub_key[u] << 32) | (uint32_t)~(uint32_t)ss.sub_idx[u]) > mine;
            take = better < need2;
        }
        takes |= (uint32_t)take << c;
    }
    int tot;
    int pos = block_scan_excl<kWG>(__popc(takes), ss.s_wave, &tot);
#pragma unroll
    for (int c = 0; c < kMaxC; ++c)
        if (takes >> c & 1u) ss.sel[pos++] = c_idx[i0 + c];
    __syncthreads();
    const int32_t *sel = ss.sel;
    for (int i = tid; i < na + need; i += kWG) {
        const bool above = i < na;
        const int32_t x = above ? v[i] : sel[i - na];
        const int32_t *other = above ? sel : v;
        int lo = 0, hi = above ? need : na;  // count of `other` below x
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (other[mid] < x) lo = mid + 1; else hi = mid;
        }
        out[(above ? i : i - na) + lo] = x;
    }
    return true;
}

}  // namespace

// ---------------------------------------------------------------------------
// Short rows: whole row in LDS.
__global__ __launch_bounds__(kWG) void topk_lds_kernel(TopkArgs a) {
    __shared__ uint32_t keys[kTopkSmallMax];
    __shared__ TopkShared sh;
    const int qi = blockIdx.x;
    topk_row<true>(a.scores + (size_t)qi * a.n_max, query_visible(a, qi), a.K, a.idx + (size_t)qi * a.K,
                   keys, sh);
}

// ---------------------------------------------------------------------------
// Histogram windows of a score row (when the scorer did not write them).
__global__ __launch_bounds__(kAuxThreads) void topk_hist_kernel(TopkArgs a) {
    __shared__ uint32_t lh[kTopkBins];
    __shared__ int s_red[4];
    const int qi = blockIdx.y;
    const int n = query_visible(a, qi);
    if (n <= a.K) return;  // the same for every workgroup of this query
    for (int i = threadIdx.x; i < kTopkBins; i += kAuxThreads) lh[i] = 0u;
    __syncthreads();
    const float *row = a.scores + (size_t)qi * a.n_max;
    const int j0 = blockIdx.x * a.hist_chunk;
    const int j1 = j0 + a.hist_chunk < n ? j0 + a.hist_chunk : n;
    for (int jb = j0; jb < j1; jb += kTopkAuxChunk) {
        float v[kPerThread];
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
            const int j = jb + k * kAuxThreads + threadIdx.x;
            v[k] = j < j1 ? row[j] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
            const int j = jb + k * kAuxThreads + threadIdx.x;
            lds_hist_add(lh, order_key(v[k]) >> 20, j < j1);
        }
    }
    const size_t w = (size_t)qi * a.n_win + blockIdx.x;
    hist_window_store(lh, a.win_hdr + w, a.win_cnt + w * kTopkWin, s_red);
}

// ---------------------------------------------------------------------------
// Scan a row into the index-ordered lists of entries above the threshold bin
// (v) and inside it (c_key, c_idx), then select.  The first round of scores
// (xa: kRound per thread, thread t taking entries kRound t ..) is loaded by the
// caller, so it can be in flight while the threshold is worked out; later rounds
// are loaded one ahead of the round being classified.  Each thread takes
// consecutive scores, so the lists come out in index order.  Returns false
// (nothing written, the same in every thread) if a list overflowed.
constexpr int kRound = 16;  // scores per thread per round
template <int NT>
struct ScanSharedT {
    int32_t v[kTopkMaxK];
    uint32_t c_key[kTopkCand];
    int32_t c_idx[kTopkCand];
    SelectSharedT<NT> ss;
};
using ScanShared = ScanSharedT<kWG>;

template <int NT = kWG>
__device__ bool scan_and_select(const float *row, int n, int n_max, bool vec, int K, uint32_t bin, float (&xa)[kRound],
                                int32_t *out, ScanSharedT<NT> &sc, int *s_red) {
    constexpr int kWG = NT;
    constexpr int kSpan = kRound * kWG;
    const int tid = threadIdx.x;
    float xb[kRound];
    int na = 0, nc = 0;
    for (int j0 = 0; j0 < n; j0 += 2 * kSpan) {
        if (j0 + kSpan < n) load_chunk<kRound>(row, j0 + kSpan + kRound * tid, n, n_max, vec, xb);
        classify_ordered<kWG, kRound>(xa, j0 + kRound * tid, n, bin, s_red, na, nc, sc.v, K, sc.c_key, sc.c_idx,
                                      kTopkCand);
        if (j0 + kSpan >= n) break;
        if (j0 + 2 * kSpan < n) load_chunk<kRound>(row, j0 + 2 * kSpan + kRound * tid, n, n_max, vec, xa);
        classify_ordered<kWG, kRound>(xb, j0 + kSpan + kRound * tid, n, bin, s_red, na, nc, sc.v, K, sc.c_key,
                                      sc.c_idx, kTopkCand);
    }
    __syncthreads();
    if (!(na < K && nc <= kTopkCand && na + nc >= K)) return false;
    return select_ordered(sc.v, na, sc.c_key, sc.c_idx, nc, K, out, sc.ss);
}

// One workgroup per query (rows up to kTopkOneKernelMax, or many queries):
// threshold from the histogram windows, scan and selection.
__global__ __launch_bounds__(kWG) void topk_onekernel_kernel(TopkArgs a) {
    __shared__ __attribute__((aligned(16))) ScanShared sc;
    __shared__ TopkShared sh;
    __shared__ uint32_t s_hist[kTopkWin];
    __shared__ int s_red[kWaves];
    const int qi = blockIdx.x;
    const int tid = threadIdx.x;
    const int n = query_visible(a, qi);
    const int K = a.K;
    const float *row = a.scores + (size_t)qi * a.n_max;
    int32_t *out = a.idx + (size_t)qi * K;
    if (n <= K) {
        for (int i = tid; i < K; i += kWG) out[i] = i < n ? i : -1;
        return;
    }
    // the first round of scores goes out together with the window loads
    const bool vec = (a.n_max & 3) == 0 && ((uintptr_t)a.scores & 15) == 0;
    float xa[kRound];
    load_chunk<kRound>(row, kRound * tid, n, a.n_max, vec, xa);
    const uint32_t bin = window_threshold(a.win_hdr + (size_t)qi * a.n_win,
                                          a.win_cnt + (size_t)qi * a.n_win * kTopkWin, a.n_win, K, s_red, s_hist);
    bool ok = bin != kNoBin && scan_and_select(row, n, a.n_max, vec, K, bin, xa, out, sc, s_red);
    if (!ok) {
        __syncthreads();
        topk_row<false>(row, n, K, out, nullptr, sh);
    }
}

// ---------------------------------------------------------------------------
// Regions for the selection after the tiled (many-query) scorer, which builds
// the histogram windows but cannot keep a chunk's keys: workgroup (chunk c,
// query) re-reads the chunk's visible scores and emits, in index order, those
// at or above the lowest bin of its window whose count from the top fits the
// region (em_cap entries), as the decode scorer emits from LDS.  A window
// whose top bin alone does not fit gets cut = top + 1 and nothing emitted
// (the selection then scans the row).  Consecutive threads take consecutive
// 8-entry runs (one 32-byte load each when the row allows), an ordered
// compaction per round.
__global__ __launch_bounds__(kAuxThreads) void topk_emit_kernel(TopkArgs a) {
    constexpr int kE = 8;
    __shared__ int s_wave[kAuxThreads / 64];
    __shared__ int s_cut;
    const int qi = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
    const int n = query_visible(a, qi);
    if (n <= a.K) return;  // the selection returns before reading regions for these
    const size_t w = (size_t)qi * a.n_win + c;
    const int cap = a.em_cap;
    if (tid < 64) {
        const int m_top = a.win_hdr[w];
        const uint32_t cnt = tid < kTopkWin ? a.win_cnt[w * kTopkWin + tid] : 0u;  // bin m_top - 31 + tid
        // suffix sums over the window (lanes kTopkWin.. hold 0)
        const uint32_t inc = wave_incl_scan_u(cnt);
        const uint32_t suf = __builtin_amdgcn_readlane(inc, 63) - inc + cnt;
        const uint64_t fits = __ballot(tid < kTopkWin && suf <= (uint32_t)cap);
        if (tid == 0)
            s_cut = m_top < 0 ? 0 : (fits ? m_top - (kTopkWin - 1) + __builtin_ctzll(fits) : m_top + 1);
    }
    __syncthreads();
    const int cut = s_cut;
    const float *row = a.scores + (size_t)qi * a.n_max;
    uint32_t *okey = a.em_key + w * cap;
    int32_t *oidx = a.em_idx + w * cap;
    const int j0 = c * a.em_chunk, j1 = min(j0 + a.em_chunk, n);
    const bool vec = (a.n_max & 3) == 0 && ((uintptr_t)a.scores & 15) == 0;
    int written = 0;
    for (int i0 = j0; i0 < j1; i0 += kAuxThreads * kE) {
        float x[kE];
        load_chunk<kE>(row, i0 + kE * tid, j1, a.n_max, vec, x);
        uint32_t k[kE];
        int m = 0;
#pragma unroll
        for (int e = 0; e < kE; ++e) {
            k[e] = order_key(x[e]);
            m += i0 + kE * tid + e < j1 && (int)(k[e] >> 20) >= cut;
        }
        int rt;
        int pos = written + block_scan_excl<kAuxThreads>(m, s_wave, &rt);
#pragma unroll
        for (int e = 0; e < kE; ++e) {
            const int j = i0 + kE * tid + e;
            if (j < j1 && (int)(k[e] >> 20) >= cut) {
                if (pos < cap) {
                    okey[pos] = k[e];
                    oidx[pos] = j;
                }
                ++pos;
            }
        }
        written += rt;
    }
    for (int i = written + tid; i < cap; i += kAuxThreads) okey[i] = 0u;
    if (tid == 0) {
        a.em_hdr[2 * w] = cut;
        a.em_hdr[2 * w + 1] = written;
    }
}

// ---------------------------------------------------------------------------
// Selection from the entries the decode scorer emitted (fused decode path).
// Per query, in one load round: the histogram windows (which give the
// threshold bin), each region's header (cut bin, count) and every emitted slot
// (regions in stretch order, each region's entries in index order, so slot
// order is index order; slot r * kWG + t goes to thread t, so each load
// instruction of a wave reads 256 contiguous bytes; the scorer zero-fills a
// region's slots past its count, and no real key is 0).  If every region's cut
// lies at or below the threshold bin, the emitted entries hold every entry at
// or above it, and the selection runs on the slots as loaded (select_slots).
// Otherwise (a region with too many high entries to emit them all) the whole
// row is scanned with the threshold instead, and without a usable threshold
// the exact radix selection runs.
constexpr int kListRounds = kTopkMaxSlots / kWG;  // rounds of kWG slots at most

// Selection straight from the slots, held in registers (slot r * kWG + tid in
// key[r], idx[r]; slot order is index order, dead slots have key 0), given the
// threshold bin: every live slot above it is taken, and of those inside it
// ("candidates") the need = K - (above) largest keys, ties to the lower index.
// A 256-bin histogram of the candidates' key bits 19..12 gives the sub-bin b2
// holding the need-th candidate and how many of b2's members (need2) are
// taken.  b2's members, when few (kSubFast at most), are gathered in LDS with
// their slot numbers and each ranks itself among them ((key, lower slot)
// order); otherwise two more radix levels (bits 11..4, 3..0) give the exact
// K-th key t and how many slots equal to t are taken.  Then one scan over the
// slots, counting per (round, wave) the slots taken outright and those equal
// to t (none on the fast path), gives each taken slot its output position:
// (taken outright before it) + min(equal before it, equal taken).  Returns
// false (nothing written, the same in every thread) if the counts are not
// those of a usable threshold.
constexpr int kSubFast = 128;  // b2 members ranked pairwise at most
__device__ bool select_slots(const uint32_t (&key)[kListRounds], const int32_t (&idx)[kListRounds], int rounds,
                             uint32_t bin, int K, int32_t *out, TopkShared &sh, uint32_t *s_base, int *s_red,
                             uint32_t *s_mkey, int *s_mslot) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    auto isum = [](int x) { return __builtin_amdgcn_readlane(wave_incl_scan(x), 63); };
    // level 1: candidates by key bits 19..12, and the count above the bin
    if (tid < 256) sh.hist[tid] = 0u;
    if (tid == 0) sh.bcast[2] = 0;  // b2 members gathered
    __syncthreads();
    int n_above = 0;
#pragma unroll
    for (int r = 0; r < kListRounds; ++r) {
        if (r < rounds) {
            const uint32_t b = key[r] >> 20;
            n_above += key[r] != 0u && b > bin;
            if (key[r] != 0u && b == bin) atomicAdd(&sh.hist[(key[r] >> 12) & 0xFFu], 1u);
        }
    }
    n_above = isum(n_above);
    if (lane == 0) s_red[wave] = n_above;
    __syncthreads();
    int na = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) na += s_red[w];
    const int need = K - na;
    if (tid < 64) {  // wave 0: the candidates' total, and the sub-bin of the need-th one (from the top)
        uint32_t h[4], sum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            h[i] = sh.hist[4 * lane + i];
            sum += h[i];
        }
        const uint32_t inc = wave_incl_scan_u(sum);
        const uint32_t total = __builtin_amdgcn_readlane(inc, 63);
        const uint32_t suf = total - inc + sum;  // over lanes >= this lane
        if (lane == 0) sh.bcast[3] = (int)total;
        if (need >= 1 && (uint32_t)need <= total) {
            uint32_t above = suf - sum;
#pragma unroll
            for (int i = 3; i >= 0; --i) {
                if (above < (uint32_t)need && (uint32_t)need <= above + h[i]) {
                    sh.bcast[0] = 4 * lane + i;
                    sh.bcast[1] = need - (int)above;
                }
                above += h[i];
            }
        }
    }
    __syncthreads();
    if (need < 1 || need > sh.bcast[3]) return false;  // the same in every thread
    const uint32_t b2 = (uint32_t)sh.bcast[0];
    int need2 = sh.bcast[1];
    const uint32_t p2 = (bin << 8) | b2;  // key bits 31..12 of the deciding candidates
    // gather b2's members (key, slot) while few
#pragma unroll
    for (int r = 0; r < kListRounds; ++r) {
        if (r < rounds && key[r] != 0u && (key[r] >> 12) == p2) {
            const int at = atomicAdd(&sh.bcast[2], 1);
            if (at < kSubFast) {
                s_mkey[at] = key[r];
                s_mslot[at] = r * kWG + tid;
            }
        }
    }
    __syncthreads();
    const int m2 = sh.bcast[2];
    uint32_t t = 0u;       // the K-th key (slow path)
    int n_eq_take = 0;     // slots equal to t taken (slow path)
    uint32_t taken2 = 0u;  // bit r: slot r * kWG + tid is a b2 member that is taken (fast path)
    if (m2 <= kSubFast) {
#pragma unroll
        for (int r = 0; r < kListRounds; ++r) {
            if (r < rounds && key[r] != 0u && (key[r] >> 12) == p2) {
                const uint64_t mine = (uint64_t)key[r] << 32 | (uint32_t)~(uint32_t)(r * kWG + tid);
                int better = 0;
                for (int u = 0; u < m2; ++u)
                    better += ((uint64_t)s_mkey[u] << 32 | (uint32_t)~(uint32_t)s_mslot[u]) > mine;
                taken2 |= (uint32_t)(better < need2) << r;
            }
        }
        t = 0xFFFFFFFFu;  // no slot is "equal to t" on this path
    } else {
        // level 2: bits 11..4 of the candidates with bits 31..12 = p2
        if (tid < 256) sh.hist[tid] = 0u;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < kListRounds; ++r)
            if (r < rounds && key[r] != 0u && (key[r] >> 12) == p2) atomicAdd(&sh.hist[(key[r] >> 4) & 0xFFu], 1u);
        __syncthreads();
        find_bin_256(sh, need2);
        __syncthreads();
        const uint32_t b3 = (uint32_t)sh.bcast[0];
        const int need3 = sh.bcast[1];
        const uint32_t p3 = (p2 << 8) | b3;  // key bits 31..4
        // level 3: bits 3..0
        __syncthreads();
        if (tid < 256) sh.hist[tid] = 0u;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < kListRounds; ++r)
            if (r < rounds && key[r] != 0u && (key[r] >> 4) == p3) atomicAdd(&sh.hist[key[r] & 0xFu], 1u);
        __syncthreads();
        find_bin_256(sh, need3);
        __syncthreads();
        t = (p3 << 4) | (uint32_t)sh.bcast[0];
        n_eq_take = sh.bcast[1];
    }
    const bool fast = m2 <= kSubFast;
    // per (round, wave): slots taken outright | slots equal to t << 16
    uint64_t m_def[kListRounds], m_eq[kListRounds];
#pragma unroll
    for (int r = 0; r < kListRounds; ++r) {
        if (r < rounds) {
            const uint32_t k = key[r];
            const bool live = k != 0u, cand = live && (k >> 20) == bin;
            const bool def = live && ((k >> 20) > bin ||
                                      (cand && (fast ? (((k >> 12) & 0xFFu) > b2 || ((taken2 >> r) & 1u)) : k > t)));
            m_def[r] = __ballot(def);
            m_eq[r] = __ballot(!fast && live && k == t);
            if (lane == 0) s_base[r * kWaves + wave] = (uint32_t)__popcll(m_def[r]) | (uint32_t)__popcll(m_eq[r]) << 16;
        }
    }
    __syncthreads();
    if (tid < 64) {  // exclusive scan of the (round, wave) counts in slot order, 2 entries per lane
        const int m = rounds * kWaves;
        uint32_t c[2], sum = 0;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            c[i] = 2 * tid + i < m ? s_base[2 * tid + i] : 0u;
            sum += c[i];
        }
        const uint32_t inc = wave_incl_scan_u(sum);
        uint32_t run = inc - sum;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (2 * tid + i < m) s_base[2 * tid + i] = run;
            run += c[i];
        }
    }
    __syncthreads();
    const uint64_t lt = lanemask_lt();
#pragma unroll
    for (int r = 0; r < kListRounds; ++r) {
        if (r < rounds) {
            const uint32_t base = s_base[r * kWaves + wave];
            const int d_before = (int)(base & 0xFFFFu) + __popcll(m_def[r] & lt);
            const int e_before = (int)(base >> 16) + __popcll(m_eq[r] & lt);
            if ((m_def[r] >> lane) & 1u) out[d_before + min(e_before, n_eq_take)] = idx[r];
            else if (((m_eq[r] >> lane) & 1u) && e_before < n_eq_take) out[d_before + e_before] = idx[r];
        }
    }
    return true;
}

// Threshold bin (key bits 31..20) of the K-th largest live slot key, from the
// slots themselves (regions that hold each chunk's K best entries: the K-th
// largest slot key is then the row's K-th largest key).  Two 256-bin levels,
// key bits 31..24 then 23..20; the live slots must number K or more.
__device__ uint32_t slots_threshold(const uint32_t (&key)[kListRounds], int rounds, int K, TopkShared &sh) {
    const int tid = threadIdx.x;
    if (tid < 256) sh.hist[tid] = 0u;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kListRounds; ++r)
        if (r < rounds) lds_hist_add(sh.hist, key[r] >> 24, key[r] != 0u);
    __syncthreads();
    find_bin_256(sh, K);
    __syncthreads();
    const uint32_t b1 = (uint32_t)sh.bcast[0];
    const int need = sh.bcast[1];
    __syncthreads();
    if (tid < 256) sh.hist[tid] = 0u;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kListRounds; ++r)
        if (r < rounds) lds_hist_add(sh.hist, (key[r] >> 20) & 0xFu, key[r] != 0u && (key[r] >> 24) == b1);
    __syncthreads();
    find_bin_256(sh, need);
    __syncthreads();
    const uint32_t bin = b1 << 4 | (uint32_t)sh.bcast[0];
    __syncthreads();
    return bin;
}

__global__ __launch_bounds__(kWG) void topk_lists_kernel(TopkArgs a) {
    __shared__ __attribute__((aligned(16))) ScanShared sc;
    __shared__ TopkShared sh;
    __shared__ uint32_t s_hist[kTopkWin];
    __shared__ int s_red[kWaves];
    __shared__ uint32_t s_base[kListRounds * kWaves];  // packed counts before each (round, wave)
    const int qi = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = a.K;
    const float *row = a.scores + (size_t)qi * a.n_max;
    int32_t *out = a.idx + (size_t)qi * K;
    const int R = a.n_win, cap = a.em_cap, slots = R * cap;
    const int rounds = (slots + kWG - 1) / kWG;  // the same in every thread
    const size_t q0 = (size_t)qi * R;
    const uint32_t *ekey = a.em_key + q0 * cap;
    const int32_t *eidx = a.em_idx + q0 * cap;
    // load round: this thread's slots, a region header, then the windows
    uint32_t key[kListRounds];
    int32_t idx[kListRounds];
#pragma unroll
    for (int r = 0; r < kListRounds; ++r) {
        if (r < rounds) {
            const int p = r * kWG + tid;
            key[r] = p < slots ? ekey[p] : 0u;
            idx[r] = p < slots ? eidx[p] : 0;
        }
    }
    int cut = 0, cnt = 0;
    if (tid < R) {
        cut = a.em_hdr[2 * (q0 + tid)];
        cnt = a.em_hdr[2 * (q0 + tid) + 1];
    }
    const int n = query_visible(a, qi);
    if (a.em_stream) {  // every region holds its chunk's K best entries
        if (n <= K) {
            for (int i = tid; i < K; i += kWG) out[i] = i < n ? i : -1;
            return;
        }
        const uint32_t bin = slots_threshold(key, rounds, K, sh);
        if (!select_slots(key, idx, rounds, bin, K, out, sh, s_base, s_red, sc.c_key, sc.c_idx))
            for (int i = tid; i < K; i += kWG) out[i] = -1;  // not reached: the slots hold the row's K best
        return;
    }
    // The windows are merged before the visible count is looked at, so their
    // loads go out in the same round as the slots and the count (a query with
    // no more than K visible entries wrote no windows and ignores the merge;
    // the reads stay inside the window arrays either way).
    const uint32_t bin = window_threshold(a.win_hdr + q0, a.win_cnt + q0 * kTopkWin, R, K, s_red, s_hist);
    if (n <= K) {
        for (int i = tid; i < K; i += kWG) out[i] = i < n ? i : -1;
        return;
    }
    // every region emitted all of its entries at or above the threshold bin?
    bool ok = bin != kNoBin && !__syncthreads_or(tid < R && ((uint32_t)cut > bin || cnt > cap));
    if (ok) ok = select_slots(key, idx, rounds, bin, K, out, sh, s_base, s_red, sc.c_key, sc.c_idx);
    if (!ok && bin != kNoBin) {  // lists not usable: scan the row with the threshold
        __syncthreads();
        const bool vec = (a.n_max & 3) == 0 && ((uintptr_t)a.scores & 15) == 0;
        float xa[kRound];
        load_chunk<kRound>(row, kRound * tid, n, a.n_max, vec, xa);
        ok = scan_and_select(row, n, a.n_max, vec, K, bin, xa, out, sc, s_red);
    }
    if (!ok) {
        __syncthreads();
        topk_row<false>(row, n, K, out, nullptr, sh);
    }
}

// ---------------------------------------------------------------------------
// Long rows: many-workgroup scan (with its own threshold merge), then selection.
// Each filter workgroup first merges the query's histogram windows into the
// threshold bin (the same result in every workgroup; its loads go out in the
// same round as the workgroup's scores), then writes its own region:
// [0] above count (0xFFFFFFFF when a list overflowed or there is no usable
// threshold), [1] candidate count, then the above list, candidate keys and
// candidate indices.
// kVec: the rows are 16-byte aligned and n_max is a multiple of kPerThread
// (whole 16-byte score loads, a thread's chunk never crosses the row end;
// decided on the host, so the loads need no branch).
template <bool kVec>
__global__ __launch_bounds__(kAuxThreads) void topk_filter_kernel(TopkArgs a) {
    __shared__ int32_t l_above[kFltAboveCap];
    __shared__ uint32_t l_ckey[kFltCandCap];
    __shared__ int32_t l_cidx[kFltCandCap];
    __shared__ int l_cnt[2];
    __shared__ uint32_t s_hist[kTopkWin];
    __shared__ int s_red[4];
    const int qi = blockIdx.y;
    const int j0 = blockIdx.x * kTopkAuxChunk;
    uint32_t *reg = a.flt + ((size_t)qi * gridDim.x + blockIdx.x) * kFltRegionWords;
    const float *row = a.scores + (size_t)qi * a.n_max;
    const int j_first = j0 + kPerThread * threadIdx.x;  // this thread's consecutive scores
    // The chunk's scores and the histogram windows are read in the same round as the
    // query's visible count (both stay inside their arrays whatever the count); the
    // scores past the count are zeroed once it is known, and a workgroup with nothing to
    // do leaves after the window merge (whose result it then ignores).
    const int seq_len = a.seq_len[qi / a.T], q_pos = a.q_pos[qi];  // read now, used after the merge
    float x[kPerThread];
    if (kVec) {  // n_max % kPerThread == 0, so a chunk starting inside the row ends inside it
        const int jf = j_first < a.n_max ? j_first : a.n_max - kPerThread;
#pragma unroll
        for (int k = 0; k < kPerThread; k += 4) {
            const float4 f = *(const float4 *)(row + jf + k);
            x[k] = f.x, x[k + 1] = f.y, x[k + 2] = f.z, x[k + 3] = f.w;
        }
    } else {
        load_chunk<kPerThread>(row, j_first, a.n_max, a.n_max, false, x);
    }
    const uint32_t bin = window_threshold(a.win_hdr + (size_t)qi * a.n_win,
                                          a.win_cnt + (size_t)qi * a.n_win * kTopkWin, a.n_win, a.K, s_red, s_hist);
    const int nv = visible_entries(seq_len, q_pos, a.ratio);
    const int n = nv < a.n_max ? nv : a.n_max;
    if (n <= a.K || j0 >= n) return;  // the selection reads regions below n only
#pragma unroll
    for (int k = 0; k < kPerThread; ++k)
        if (j_first + k >= n) x[k] = 0.f;
    if (bin == kNoBin) {
        if (threadIdx.x == 0) reg[0] = 0xFFFFFFFFu;
        return;
    }
    // lists in index order, so the selection can merge them without sorting
    int n_gt = 0, n_eq = 0;
    classify_ordered<kAuxThreads, kPerThread>(x, j_first, n, bin, s_red, n_gt, n_eq, l_above, kFltAboveCap, l_ckey,
                                              l_cidx, kFltCandCap);
    if (threadIdx.x == 0) {
        l_cnt[0] = n_gt;
        l_cnt[1] = n_eq;
    }
    __syncthreads();
    const int na = l_cnt[0], nc = l_cnt[1];
    const bool over = na > kFltAboveCap || nc > kFltCandCap;
    if (threadIdx.x == 0) {
        reg[0] = over ? 0xFFFFFFFFu : (uint32_t)na;
        reg[1] = (uint32_t)nc;
    }
    if (over) return;
    for (int i = threadIdx.x; i < na; i += kAuxThreads) reg[2 + i] = (uint32_t)l_above[i];
    for (int i = threadIdx.x; i < nc; i += kAuxThreads) {
        reg[2 + kFltAboveCap + i] = l_ckey[i];
        reg[2 + kFltAboveCap + kFltCandCap + i] = (uint32_t)l_cidx[i];
    }
}

__global__ __launch_bounds__(kWG) void topk_final_kernel(TopkArgs a, int n_flt) {
    __shared__ __attribute__((aligned(16))) int32_t v[kTopkMaxK];
    __shared__ uint32_t c_key[kTopkCand];
    __shared__ int32_t c_idx[kTopkCand];
    __shared__ SelectShared ss;
    __shared__ TopkShared sh;
    __shared__ int s_bad;
    const int qi = blockIdx.x;
    const int tid = threadIdx.x;
    const int K = a.K;
    const float *row = a.scores + (size_t)qi * a.n_max;
    int32_t *out = a.idx + (size_t)qi * K;
    // Gather the filter lists of the workgroups that covered visible entries,
    // kFinalGroup threads per region.  One round loads every header together
    // with the first entries of each list (lists are short: a few entries per
    // region in practice); whatever lies beyond takes one more round.  The
    // first pass's loads go out with the query's visible count (they stay
    // inside the regions this launch has; regions past the count are ignored).
    const uint32_t *reg0 = a.flt + (size_t)qi * n_flt * kFltRegionWords;
    constexpr int kRegPer = kWG / kFinalGroup;  // regions per pass
    const int u = tid % kFinalGroup;
    struct RegionHead {
        uint32_t na, nc, sa, sck[kSpecC], sci[kSpecC];
    };
    auto load_head = [&](int r, RegionHead &h) {
        const uint32_t *reg = reg0 + (size_t)r * kFltRegionWords;
        h.na = reg[0];
        h.nc = reg[1];
        h.sa = reg[2 + u];
#pragma unroll
        for (int k = 0; k < kSpecC; ++k) {
            h.sck[k] = reg[2 + kFltAboveCap + u + kFinalGroup * k];
            h.sci[k] = reg[2 + kFltAboveCap + kFltCandCap + u + kFinalGroup * k];
        }
    };
    RegionHead h0;
    load_head(min(tid / kFinalGroup, n_flt - 1), h0);
    const int n = query_visible(a, qi);
    if (n <= K) {
        for (int i = tid; i < K; i += kWG) out[i] = i < n ? i : -1;
        return;
    }
    bool ok = true;
    if (tid == 0) s_bad = 0;
    __syncthreads();
    const int n_reg = (n + kTopkAuxChunk - 1) / kTopkAuxChunk;
    int na_tot = 0, nc_tot = 0;
    for (int r0 = 0; r0 < n_reg; r0 += kRegPer) {
        const int r = r0 + tid / kFinalGroup;
        const bool live = r < n_reg;
        RegionHead hd;
        if (r0 == 0)
            hd = h0;
        else
            load_head(live ? r : r0, hd);
        const uint32_t *reg = reg0 + (size_t)(live ? r : r0) * kFltRegionWords;
        uint32_t na = hd.na, nc = hd.nc;
        if (!live) na = nc = 0;
        if (na > (uint32_t)kFltAboveCap || nc > (uint32_t)kFltCandCap) {
            s_bad = 1;  // overflowed or unusable region: the exact path runs
            na = nc = 0;
        }
        int tot;
        const int pre = block_scan_excl<kWG>(u == 0 ? (int)(na | (nc << 16)) : 0, ss.s_wave, &tot);
        // this region's list offsets: the scan value of its first thread
        const int base = __shfl(pre, (tid & 63) & ~(kFinalGroup - 1));
        const int pa = na_tot + (base & 0xFFFF), pc = nc_tot + (base >> 16);
        if ((uint32_t)u < na && pa + u < K) v[pa + u] = (int32_t)hd.sa;
#pragma unroll
        for (int k = 0; k < kSpecC; ++k) {
            const int i = u + kFinalGroup * k;
            if ((uint32_t)i < nc && pc + i < kTopkCand) {
                c_key[pc + i] = hd.sck[k];
                c_idx[pc + i] = (int32_t)hd.sci[k];
            }
        }
        for (int i = kFinalGroup + u; i < (int)na; i += kFinalGroup)  // beyond the first round
            if (pa + i < K) v[pa + i] = (int32_t)reg[2 + i];
        for (int i = kFinalGroup * kSpecC + u; i < (int)nc; i += kFinalGroup)
            if (pc + i < kTopkCand) {
                c_key[pc + i] = reg[2 + kFltAboveCap + i];
                c_idx[pc + i] = (int32_t)reg[2 + kFltAboveCap + kFltCandCap + i];
            }
        na_tot += tot & 0xFFFF;
        nc_tot += tot >> 16;
    }
    __syncthreads();
    ok = ok && !s_bad && na_tot < K && nc_tot <= kTopkCand && na_tot + nc_tot >= K;
    if (ok) {  // the regions' lists are in index order, and so are their concatenations
        ok = select_ordered(v, na_tot, c_key, c_idx, nc_tot, K, out, ss);
    }
    if (!ok) {
        __syncthreads();
        topk_row<false>(row, n, K, out, nullptr, sh);
    }
}

// ---------------------------------------------------------------------------
bool topk_uses_histogram(int n_max) { return n_max > kTopkSmallMax; }

static int n_filters(int n_max) { return (n_max + kTopkAuxChunk - 1) / kTopkAuxChunk; }
// One selecting workgroup per query (no filter kernel) for rows that fit its
// scan, and whenever there are enough queries to fill the GPU that way.
static bool one_kernel(int n_max, int n_queries) {
    return n_max <= kTopkOneKernelMax || n_queries >= kTopkManyQueries;
}
// Histogram windows per query: the scorer's workgroups when it builds them,
// else one per 2,048-entry chunk, fewer (longer chunks) when many queries
// already fill the GPU.
static int n_windows(int n_max, int n_win, int n_queries) {
    if (n_win > 0) return n_win;
    int nw = n_filters(n_max);
    if (n_queries >= kTopkManyQueries) {
        const int want = 8192 / n_queries > 1 ? 8192 / n_queries : 1;
        nw = nw < want ? nw : want;
    }
    return nw;
}
static int hist_chunk(int n_max, int nw) {
    const int per = (n_max + nw - 1) / nw;
    return (per + kTopkAuxChunk - 1) / kTopkAuxChunk * kTopkAuxChunk;
}

size_t topk_workspace_bytes(int n_queries, int K, int n_max, int n_win, int em_cap) {
    (void)K;
    if (!topk_uses_histogram(n_max)) return 0;
    const size_t Q = (size_t)n_queries;
    const size_t nw = (size_t)n_windows(n_max, n_win, n_queries);
    size_t b = Q * nw * 4 + Q * nw * kTopkWin * 4 + Q * 4 + 4 * 256;
    if (em_cap > 0) {
        b += Q * nw * (2 + 2 * (size_t)em_cap) * 4 + 3 * 256;
    } else if (!one_kernel(n_max, n_queries)) {
        b += Q * (size_t)n_filters(n_max) * kFltRegionWords * 4;
    }
    return b;
}

static inline char *align256(char *p) { return (char *)(((uintptr_t)p + 255) & ~(uintptr_t)255); }

void topk_carve(TopkArgs &a, void *ws, int n_queries, int n_win, int em_cap) {
    a.n_win = n_windows(a.n_max, n_win, n_queries);
    a.hist_chunk = hist_chunk(a.n_max, a.n_win);
    a.em_cap = 0;
    if (!topk_uses_histogram(a.n_max)) return;
    const size_t Q = (size_t)n_queries;
    char *p = align256((char *)ws);
    a.win_hdr = (int32_t *)p;
    p = align256(p + Q * a.n_win * 4);
    a.win_cnt = (uint32_t *)p;
    p = align256(p + Q * a.n_win * kTopkWin * 4);
    a.bin = (uint32_t *)p;
    p = align256(p + Q * 4);
    a.flt = (uint32_t *)p;
    if (em_cap > 0) {  // the emitted regions take the place of the filter lists
        a.em_cap = em_cap;
        a.em_hdr = (int32_t *)p;
        p = align256(p + Q * a.n_win * 2 * 4);
        a.em_key = (uint32_t *)p;
        p = align256(p + Q * a.n_win * (size_t)em_cap * 4);
        a.em_idx = (int32_t *)p;
    }
}

hipError_t launch_topk(const TopkArgs &a, hipStream_t stream, bool hist_done) {
    const int Q = a.B * a.T;
    if (!topk_uses_histogram(a.n_max)) {
        hipLaunchKernelGGL(topk_lds_kernel, dim3(Q), dim3(kWG), 0, stream, a);
        return hipGetLastError();
    }
    if (a.em_cap > 0) {  // the scorer wrote the windows (or streamed its regions) and (or, em_chunk > 0, the top-k now) the regions
        if (a.em_chunk > 0) hipLaunchKernelGGL(topk_emit_kernel, dim3(a.n_win, Q), dim3(kAuxThreads), 0, stream, a);
        hipLaunchKernelGGL(topk_lists_kernel, dim3(Q), dim3(kWG), 0, stream, a);
        return hipGetLastError();
    }
    if (!hist_done) hipLaunchKernelGGL(topk_hist_kernel, dim3(a.n_win, Q), dim3(kAuxThreads), 0, stream, a);
    if (one_kernel(a.n_max, Q)) {
        hipLaunchKernelGGL(topk_onekernel_kernel, dim3(Q), dim3(kWG), 0, stream, a);
        return hipGetLastError();
    }
    const int nf = n_filters(a.n_max);
    if (a.n_max % kPerThread == 0 && ((uintptr_t)a.scores & 15) == 0)
        hipLaunchKernelGGL(topk_filter_kernel<true>, dim3(nf, Q), dim3(kAuxThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(topk_filter_kernel<false>, dim3(nf, Q), dim3(kAuxThreads), 0, stream, a);
    hipLaunchKernelGGL(topk_final_kernel, dim3(Q), dim3(kWG), 0, stream, a, nf);
    return hipGetLastError();
}

}  // namespace csa
