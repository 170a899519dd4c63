// Per-query top-k over the indexer scores (DeepSeek-V4-Flash config:
// index_topk 512; "DeepSeek-V4 Architecture Analysis", INNOVATIONS 1, indexer
// bullet).  Order is (fp32 score desc, index asc); the K chosen indices are
// written ascending, padded with -1 when fewer than K entries are visible.
//
// Scores become order-preserving uint32 keys.  Two paths:
//  * rows up to kTopkLdsCap entries: one 1024-thread workgroup per query keeps
//    the row in LDS, finds the exact K-th key with four 8-bit radix passes,
//    then writes the selection in index order with an ordered compaction
//    (wave ballots + cross-wave prefix counts), taking equal keys by index.
//  * longer rows: many workgroups per query build a 12-bit key histogram (or
//    the scorer builds it while writing the scores); the last workgroup of
//    each query locates the bin holding the K-th key.  Many workgroups then
//    copy out the entries above that bin and the candidates inside it.  One
//    workgroup per query refines the candidates with a second 12-bit
//    histogram, breaks the remaining ties by (key, -index), and writes the K
//    indices in ascending order through an LDS bitmap.  Before using the
//    candidates it checks that the counts are consistent (entries above the
//    bin < K <= above + candidates, every candidate kept); otherwise it runs
//    the exact one-workgroup scan of the whole row.  Correctness therefore
//    never depends on the workspace's prior contents; the kernels leave the
//    histogram and counters zero-filled, which makes the next call fast.
#include "common.hpp"
#include "launch.hpp"
#include "topk_hist.hpp"

namespace csa {

namespace {
constexpr int kWG = 1024;
constexpr int kWaves = kWG / 64;
constexpr int kAuxThreads = 256;

struct TopkShared {
    uint32_t hist[256];
    uint64_t masks[2][kWaves][2];
    int bcast[2];
    int count;
};

// Wave 0 finds the histogram bin that holds the need-th largest element
// (counting from bin 255 down) and publishes (bin, rank within the bin).
__device__ __forceinline__ void find_bin_256(TopkShared &sh, int need) {
    const int lane = threadIdx.x & 63;
    if (threadIdx.x < 64) {
        uint32_t h[4];
        uint32_t s = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            h[i] = sh.hist[4 * lane + i];
            s += h[i];
        }
        uint32_t suf = s;  // sum over lanes >= this lane
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t t = __shfl_down(suf, o);
            if (lane + o < 64) suf += t;
        }
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

// Exact top-k of one row (n visible entries) by one 1024-thread workgroup.
template <bool kInLds>
__device__ void topk_row(const float *__restrict__ row, int n, int K, int32_t *__restrict__ out,
                         uint32_t *keys, TopkShared &sh) {
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
        for (int i = tid; i < n; i += kWG) {
            const uint32_t k = key_at(i);
            if ((k & hi_mask) == prefix) atomicAdd(&sh.hist[(k >> shift) & 255u], 1u);
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

}  // namespace

__global__ __launch_bounds__(kWG) void topk_lds_kernel(TopkArgs a) {
    __shared__ uint32_t keys[kTopkSmallMax];
    __shared__ TopkShared sh;
    const int qi = blockIdx.x;
    topk_row<true>(a.scores + (size_t)qi * a.n_max, query_visible(a, qi), a.K, a.idx + (size_t)qi * a.K,
                   keys, sh);
}

// ---------------------------------------------------------------------------
// Multi-workgroup path.

namespace {
constexpr int kPerThread = kTopkAuxChunk / kAuxThreads;  // 8 scores per thread
constexpr int kSubCap = 1024;                            // second-level tie candidates
constexpr int kBitmapMaxN = 262144;                      // LDS bitmap ordering up to this row length
}  // namespace

__global__ __launch_bounds__(kAuxThreads) void topk_hist_kernel(TopkArgs a) {
    __shared__ uint32_t lh[kTopkBins];
    __shared__ int s_flag;
    __shared__ uint32_t s_wsum[4];
    const int qi = blockIdx.y;
    const int n = query_visible(a, qi);
    if (n <= a.K) return;  // the same for every workgroup of this query
    hist_begin(a.ctrl + (size_t)qi * kTopkCtrl);
    for (int i = threadIdx.x; i < kTopkBins; i += kAuxThreads) lh[i] = 0u;
    __syncthreads();
    const float *row = a.scores + (size_t)qi * a.n_max;
    const int j0 = blockIdx.x * kTopkAuxChunk + kPerThread * threadIdx.x;
    float v[kPerThread];
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) v[k] = j0 + k < n ? row[j0 + k] : 0.f;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k)
        if (j0 + k < n) atomicAdd(&lh[order_key(v[k]) >> 20], 1u);
    hist_publish(lh, a.hist + (size_t)qi * kTopkBins, a.ctrl + (size_t)qi * kTopkCtrl, n, a.K, gridDim.x,
                 &s_flag, s_wsum);
}

// Entries whose 12-bit key digit is above the threshold bin -> sel[], inside
// it -> candidates.  Slots are reserved with one atomic per list per
// workgroup; every write is bounded by its buffer.
__global__ __launch_bounds__(kAuxThreads) void topk_filter_kernel(TopkArgs a) {
    __shared__ int32_t l_sel[kTopkAuxChunk];
    __shared__ int32_t l_cidx[kTopkAuxChunk];
    __shared__ uint32_t l_ckey[kTopkAuxChunk];
    __shared__ int l_cnt[2];
    __shared__ int l_base[2];
    const int qi = blockIdx.y;
    const int n = query_visible(a, qi);
    if (n <= a.K) return;
    uint32_t *ctrl = a.ctrl + (size_t)qi * kTopkCtrl;
    const uint32_t bin = ctrl[kCtrlBin];
    if (bin >= (uint32_t)kTopkBins) return;
    if (threadIdx.x < 2) l_cnt[threadIdx.x] = 0;
    __syncthreads();
    const float *row = a.scores + (size_t)qi * a.n_max;
    const int j0 = blockIdx.x * kTopkAuxChunk + kPerThread * threadIdx.x;
    float v[kPerThread];
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) v[k] = j0 + k < n ? row[j0 + k] : 0.f;
    const uint64_t lt = lanemask_lt();
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const int j = j0 + k;
        const uint32_t key = order_key(v[k]);
        const uint32_t d = key >> 20;
        const bool gt = j < n && d > bin;
        const bool eq = j < n && d == bin;
        const uint64_t mg = __ballot(gt), me = __ballot(eq);
        if (mg) {
            int base = 0;
            if (lane == 0) base = atomicAdd(&l_cnt[0], __popcll(mg));
            base = __shfl(base, 0);
            if (gt) l_sel[base + __popcll(mg & lt)] = j;
        }
        if (me) {
            int base = 0;
            if (lane == 0) base = atomicAdd(&l_cnt[1], __popcll(me));
            base = __shfl(base, 0);
            if (eq) {
                l_cidx[base + __popcll(me & lt)] = j;
                l_ckey[base + __popcll(me & lt)] = key;
            }
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        l_base[0] = l_cnt[0] ? (int)atomicAdd(&ctrl[kCtrlAbove], (uint32_t)l_cnt[0]) : 0;
        l_base[1] = l_cnt[1] ? (int)atomicAdd(&ctrl[kCtrlCand], (uint32_t)l_cnt[1]) : 0;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < l_cnt[0]; i += kAuxThreads) {
        const int slot = l_base[0] + i;
        if (slot < a.K) a.sel[(size_t)qi * a.K + slot] = l_sel[i];
    }
    for (int i = threadIdx.x; i < l_cnt[1]; i += kAuxThreads) {
        const int slot = l_base[1] + i;
        if (slot < kTopkCand) {
            a.cand_idx[(size_t)qi * kTopkCand + slot] = l_cidx[i];
            a.cand_key[(size_t)qi * kTopkCand + slot] = l_ckey[i];
        }
    }
}

namespace {
// Block-wide exclusive prefix sum over 1024 threads (one value each).
__device__ __forceinline__ int block_exclusive_scan(int x, int *s_wave, int *total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int inc = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(inc, o);
        if (lane >= o) inc += t;
    }
    if (lane == 63) s_wave[wave] = inc;
    __syncthreads();
    int before = 0, all = 0;
    for (int w = 0; w < kWaves; ++w) {
        const int c = s_wave[w];
        before += w < wave ? c : 0;
        all += c;
    }
    __syncthreads();
    *total = all;
    return before + inc - x;
}
}  // namespace

// One workgroup per query: candidates -> exact selection -> ascending output.
__global__ __launch_bounds__(kWG) void topk_final_kernel(TopkArgs a) {
    __shared__ uint32_t c_key[kTopkCand];
    __shared__ int32_t c_idx[kTopkCand];
    __shared__ uint32_t bits[kBitmapMaxN / 32];  // also the second-level histogram
    __shared__ uint32_t sub_key[kSubCap];
    __shared__ int32_t sub_idx[kSubCap];
    __shared__ int32_t v[kTopkMaxK];
    __shared__ TopkShared sh;
    __shared__ int s_wave[kWaves];
    __shared__ int s_cnt[2];
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
    uint32_t *ctrl = a.ctrl + (size_t)qi * kTopkCtrl;
    const uint32_t bin = ctrl[kCtrlBin];
    const int n_above = (int)ctrl[kCtrlAbove];
    const int n_cand = (int)ctrl[kCtrlCand];
    __syncthreads();
    if (tid == 0) {  // leave the counters zero-filled for the next call
        ctrl[kCtrlDone] = 0u;
        ctrl[kCtrlAbove] = 0u;
        ctrl[kCtrlCand] = 0u;
    }
    const int need = K - n_above;
    const bool fast = bin < (uint32_t)kTopkBins && n_above >= 0 && n_above < K && n_cand <= kTopkCand &&
                      n_above + n_cand >= K;
    if (!fast) {
        topk_row<false>(row, n, K, out, nullptr, sh);
        return;
    }
    uint32_t *h2 = bits;  // 4096-bin histogram of key bits [19:8]
    for (int i = tid; i < kTopkBins; i += kWG) h2[i] = 0u;
    if (tid < 2) s_cnt[tid] = 0;
    for (int i = tid; i < n_above; i += kWG) v[i] = a.sel[(size_t)qi * K + i];
    for (int i = tid; i < n_cand; i += kWG) {
        c_key[i] = a.cand_key[(size_t)qi * kTopkCand + i];
        c_idx[i] = a.cand_idx[(size_t)qi * kTopkCand + i];
    }
    __syncthreads();
    for (int i = tid; i < n_cand; i += kWG) atomicAdd(&h2[(c_key[i] >> 8) & 0xFFFu], 1u);
    __syncthreads();
    // bin b2 of the need-th largest candidate: 4 bins per thread, suffix sums
    uint32_t hh[4], s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        hh[i] = h2[4 * tid + i];
        s += hh[i];
    }
    int tot;
    const int pre = block_exclusive_scan((int)s, s_wave, &tot);  // bins below this thread
    const int above_me = tot - pre - (int)s;                       // bins above this thread
    if (above_me < need && need <= above_me + (int)s) {
        int acc = above_me;
        for (int i = 3; i >= 0; --i) {
            if (acc < need && need <= acc + (int)hh[i]) {
                sh.bcast[0] = 4 * tid + i;
                sh.bcast[1] = need - acc;
                break;
            }
            acc += (int)hh[i];
        }
    }
    __syncthreads();
    const uint32_t b2 = (uint32_t)sh.bcast[0];
    const int need2 = sh.bcast[1];
    // above b2: selected; inside b2: ties to resolve by (key, -index)
    for (int i = tid; i < n_cand; i += kWG) {
        const uint32_t d2 = (c_key[i] >> 8) & 0xFFFu;
        if (d2 > b2) {
            const int slot = n_above + atomicAdd(&s_cnt[0], 1);
            if (slot < K) v[slot] = c_idx[i];
        } else if (d2 == b2) {
            const int slot = atomicAdd(&s_cnt[1], 1);
            if (slot < kSubCap) {
                sub_key[slot] = c_key[i];
                sub_idx[slot] = c_idx[i];
            }
        }
    }
    __syncthreads();
    const int n_hi = s_cnt[0], m2 = s_cnt[1];
    if (m2 > kSubCap || n_above + n_hi + need2 != K) {  // not expected; stay exact
        __syncthreads();
        topk_row<false>(row, n, K, out, nullptr, sh);
        return;
    }
    for (int t = tid; t < m2; t += kWG) {
        const uint64_t mine = ((uint64_t)sub_key[t] << 32) | (uint32_t)~(uint32_t)sub_idx[t];
        int rank = 0;
        for (int u = 0; u < m2; ++u) {
            const uint64_t other = ((uint64_t)sub_key[u] << 32) | (uint32_t)~(uint32_t)sub_idx[u];
            rank += other > mine;
        }
        if (rank < need2) v[n_above + n_hi + rank] = sub_idx[t];
    }
    __syncthreads();
    // ascending order
    if (n <= kBitmapMaxN) {
        const int n_words = (n + 31) >> 5;
        for (int i = tid; i < n_words; i += kWG) bits[i] = 0u;
        __syncthreads();
        for (int i = tid; i < K; i += kWG) atomicOr(&bits[v[i] >> 5], 1u << (v[i] & 31));
        __syncthreads();
        constexpr int kWordsPerThread = kBitmapMaxN / 32 / kWG;  // 8
        uint32_t wv[kWordsPerThread];
        int cnt = 0;
#pragma unroll
        for (int k = 0; k < kWordsPerThread; ++k) {
            const int wi = kWordsPerThread * tid + k;
            wv[k] = wi < n_words ? bits[wi] : 0u;
            cnt += __popc(wv[k]);
        }
        int pos = block_exclusive_scan(cnt, s_wave, &tot);
#pragma unroll
        for (int k = 0; k < kWordsPerThread; ++k) {
            uint32_t w = wv[k];
            while (w) {
                const int b = __ffs(w) - 1;
                if (pos < K) out[pos] = 32 * (kWordsPerThread * tid + k) + b;
                ++pos;
                w &= w - 1u;
            }
        }
    } else {
        int P = 1;
        while (P < K) P <<= 1;
        for (int i = K + tid; i < P; i += kWG) v[i] = 0x7FFFFFFF;
        __syncthreads();
        for (int size = 2; size <= P; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int t = tid; t < P / 2; t += kWG) {
                    const int i = (t / stride) * stride * 2 + (t % stride);
                    const int j = i + stride;
                    const bool asc = (i & size) == 0;
                    const int32_t x = v[i], y = v[j];
                    if ((x > y) == asc) {
                        v[i] = y;
                        v[j] = x;
                    }
                }
                __syncthreads();
            }
        }
        for (int i = tid; i < K; i += kWG) out[i] = v[i];
    }
}

bool topk_uses_histogram(int n_max) { return n_max > kTopkSmallMax; }

size_t topk_workspace_bytes(int n_queries, int K, int n_max) {
    if (!topk_uses_histogram(n_max)) return 0;
    const size_t Q = (size_t)n_queries;
    return Q * kTopkBins * 4 + Q * kTopkCtrl * 4 + Q * (size_t)K * 4 + Q * kTopkCand * 8 + 256;
}

static inline char *align256(char *p) { return (char *)(((uintptr_t)p + 255) & ~(uintptr_t)255); }

void topk_carve(TopkArgs &a, void *ws, int n_queries) {
    if (!topk_uses_histogram(a.n_max)) return;
    const size_t Q = (size_t)n_queries;
    char *p = align256((char *)ws);
    a.hist = (uint32_t *)p;
    p += Q * kTopkBins * 4;
    a.ctrl = (uint32_t *)p;
    p += Q * kTopkCtrl * 4;
    a.sel = (int32_t *)p;
    p += Q * (size_t)a.K * 4;
    a.cand_key = (uint32_t *)p;
    p += Q * kTopkCand * 4;
    a.cand_idx = (int32_t *)p;
}

hipError_t launch_topk(const TopkArgs &a, hipStream_t stream, bool hist_done) {
    const int Q = a.B * a.T;
    if (!topk_uses_histogram(a.n_max)) {
        hipLaunchKernelGGL(topk_lds_kernel, dim3(Q), dim3(kWG), 0, stream, a);
        return hipGetLastError();
    }
    const int n_chunks = (a.n_max + kTopkAuxChunk - 1) / kTopkAuxChunk;
    if (!hist_done) hipLaunchKernelGGL(topk_hist_kernel, dim3(n_chunks, Q), dim3(kAuxThreads), 0, stream, a);
    hipLaunchKernelGGL(topk_filter_kernel, dim3(n_chunks, Q), dim3(kAuxThreads), 0, stream, a);
    hipLaunchKernelGGL(topk_final_kernel, dim3(Q), dim3(kWG), 0, stream, a);
    return hipGetLastError();
}

}  // namespace csa
