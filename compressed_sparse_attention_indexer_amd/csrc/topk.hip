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
//  * longer rows: many workgroups per query build a 12-bit key histogram,
//    one small kernel locates the bin holding the K-th key, many workgroups
//    copy out the entries above that bin and the candidates inside it, and a
//    final workgroup selects among the candidates by (key, -index) and sorts
//    the K indices.  If the bin is larger than the candidate buffer, the final
//    workgroup falls back to the exact one-workgroup scan of the whole row.
#include "common.hpp"
#include "launch.hpp"

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
    __shared__ uint32_t keys[kTopkLdsCap];
    __shared__ TopkShared sh;
    const int qi = blockIdx.x;
    topk_row<true>(a.scores + (size_t)qi * a.n_max, query_visible(a, qi), a.K, a.idx + (size_t)qi * a.K,
                   keys, sh);
}

// ---------------------------------------------------------------------------
// Multi-workgroup path.

__global__ __launch_bounds__(kAuxThreads) void topk_clear_kernel(TopkArgs a, int n_queries) {
    const size_t n_hist = (size_t)n_queries * kTopkBins;
    const size_t n_cnt = (size_t)n_queries * 4;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n_hist + n_cnt;
         i += (size_t)gridDim.x * blockDim.x) {
        if (i < n_hist)
            a.hist[i] = 0u;
        else
            a.counters[i - n_hist] = 0u;
    }
}

__global__ __launch_bounds__(kAuxThreads) void topk_hist_kernel(TopkArgs a) {
    __shared__ uint32_t lh[kTopkBins];
    const int qi = blockIdx.y;
    const int n = query_visible(a, qi);
    if (n <= a.K) return;
    for (int i = threadIdx.x; i < kTopkBins; i += kAuxThreads) lh[i] = 0u;
    __syncthreads();
    const float *row = a.scores + (size_t)qi * a.n_max;
    const int j0 = blockIdx.x * a.chunk;
    const int j1 = j0 + a.chunk < n ? j0 + a.chunk : n;
    for (int j = j0 + threadIdx.x; j < j1; j += kAuxThreads) atomicAdd(&lh[order_key(row[j]) >> 20], 1u);
    __syncthreads();
    uint32_t *gh = a.hist + (size_t)qi * kTopkBins;
    for (int i = threadIdx.x; i < kTopkBins; i += kAuxThreads)
        if (lh[i]) atomicAdd(&gh[i], lh[i]);
}

// counters[q] = {threshold bin, rank needed inside it, #above, #candidates}
__global__ __launch_bounds__(kAuxThreads) void topk_thresh_kernel(TopkArgs a) {
    __shared__ uint32_t wsum[kAuxThreads / 64];
    const int qi = blockIdx.x;
    const int n = query_visible(a, qi);
    if (n <= a.K) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int kPer = kTopkBins / kAuxThreads;  // 16 bins per thread
    const uint32_t *gh = a.hist + (size_t)qi * kTopkBins;
    uint32_t h[kPer];
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        h[i] = gh[kPer * tid + i];
        s += h[i];
    }
    uint32_t suf = s;  // suffix sum within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_down(suf, o);
        if (lane + o < 64) suf += t;
    }
    if (lane == 0) wsum[wave] = suf;
    __syncthreads();
    for (int w = wave + 1; w < kAuxThreads / 64; ++w) suf += wsum[w];
    const uint32_t above = suf - s;
    const uint32_t need = (uint32_t)a.K;
    if (above < need && need <= suf) {
        uint32_t acc = above;
        for (int i = kPer - 1; i >= 0; --i) {
            if (acc < need && need <= acc + h[i]) {
                a.counters[(size_t)qi * 4 + 0] = (uint32_t)(kPer * tid + i);
                a.counters[(size_t)qi * 4 + 1] = need - acc;
                break;
            }
            acc += h[i];
        }
    }
}

__global__ __launch_bounds__(kAuxThreads) void topk_filter_kernel(TopkArgs a) {
    constexpr int kMaxChunk = 2048;
    __shared__ int32_t l_sel[kMaxChunk];
    __shared__ int32_t l_cidx[kMaxChunk];
    __shared__ uint32_t l_ckey[kMaxChunk];
    __shared__ int l_cnt[2];
    __shared__ int l_base[2];
    const int qi = blockIdx.y;
    const int n = query_visible(a, qi);
    if (n <= a.K) return;
    const uint32_t bin = a.counters[(size_t)qi * 4 + 0];
    if (threadIdx.x < 2) l_cnt[threadIdx.x] = 0;
    __syncthreads();
    const float *row = a.scores + (size_t)qi * a.n_max;
    const int j0 = blockIdx.x * a.chunk;
    const int j1 = j0 + a.chunk < n ? j0 + a.chunk : n;
    const uint64_t lt = lanemask_lt();
    const int lane = threadIdx.x & 63;
    for (int jb = j0; jb < j1; jb += kAuxThreads) {
        const int j = jb + threadIdx.x;
        const uint32_t k = j < j1 ? order_key(row[j]) : 0u;
        const uint32_t d = k >> 20;
        const bool gt = j < j1 && d > bin;
        const bool eq = j < j1 && d == bin;
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
                l_ckey[base + __popcll(me & lt)] = k;
            }
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        l_base[0] = l_cnt[0] ? (int)atomicAdd(&a.counters[(size_t)qi * 4 + 2], (uint32_t)l_cnt[0]) : 0;
        l_base[1] = l_cnt[1] ? (int)atomicAdd(&a.counters[(size_t)qi * 4 + 3], (uint32_t)l_cnt[1]) : 0;
    }
    __syncthreads();
    // entries above the threshold bin: fewer than K in total
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

__global__ __launch_bounds__(kWG) void topk_final_kernel(TopkArgs a) {
    __shared__ uint32_t c_key[kTopkCand];
    __shared__ uint32_t c_nidx[kTopkCand];  // ~index: larger means lower index
    __shared__ int32_t v[kTopkMaxK];
    __shared__ TopkShared sh;
    const int qi = blockIdx.x;
    const int tid = threadIdx.x;
    const int n = query_visible(a, qi);
    const float *row = a.scores + (size_t)qi * a.n_max;
    int32_t *out = a.idx + (size_t)qi * a.K;
    if (n <= a.K) {
        for (int i = tid; i < a.K; i += kWG) out[i] = i < n ? i : -1;
        return;
    }
    const int need0 = (int)a.counters[(size_t)qi * 4 + 1];
    const int n_above = (int)a.counters[(size_t)qi * 4 + 2];
    const int n_cand = (int)a.counters[(size_t)qi * 4 + 3];
    if (n_cand > kTopkCand || n_above + need0 != a.K) {  // bin too large: exact whole-row scan
        topk_row<false>(row, n, a.K, out, nullptr, sh);
        return;
    }
    for (int i = tid; i < n_cand; i += kWG) {
        c_key[i] = a.cand_key[(size_t)qi * kTopkCand + i];
        c_nidx[i] = ~(uint32_t)a.cand_idx[(size_t)qi * kTopkCand + i];
    }
    for (int i = tid; i < n_above; i += kWG) v[i] = a.sel[(size_t)qi * a.K + i];
    if (tid == 0) sh.count = 0;
    __syncthreads();
    // need0-th largest composite (key, ~index) among the candidates; composites are unique.
    uint64_t prefix = 0;
    int need = need0;
    for (int pass = 0; pass < 8; ++pass) {
        const int shift = 56 - 8 * pass;
        const uint64_t hi_mask = pass == 0 ? 0ull : (~0ull << (shift + 8));
        if (tid < 256) sh.hist[tid] = 0;
        __syncthreads();
        for (int i = tid; i < n_cand; i += kWG) {
            const uint64_t c = ((uint64_t)c_key[i] << 32) | c_nidx[i];
            if ((c & hi_mask) == prefix) atomicAdd(&sh.hist[(c >> shift) & 255u], 1u);
        }
        __syncthreads();
        find_bin_256(sh, need);
        __syncthreads();
        prefix |= (uint64_t)sh.bcast[0] << shift;
        need = sh.bcast[1];
        __syncthreads();
    }
    for (int i = tid; i < n_cand; i += kWG) {
        const uint64_t c = ((uint64_t)c_key[i] << 32) | c_nidx[i];
        if (c >= prefix) {
            const int slot = atomicAdd(&sh.count, 1);
            if (slot < need0) v[n_above + slot] = (int32_t)~c_nidx[i];
        }
    }
    // bitonic sort of the K indices (padded to a power of two)
    int P = 1;
    while (P < a.K) P <<= 1;
    __syncthreads();
    for (int i = a.K + tid; i < P; i += kWG) v[i] = 0x7FFFFFFF;
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
    for (int i = tid; i < a.K; i += kWG) out[i] = v[i];
}

size_t topk_workspace_bytes(int n_queries, int K, int n_max) {
    if (n_max <= kTopkLdsCap) return 0;
    const size_t Q = (size_t)n_queries;
    return Q * kTopkBins * 4 + Q * 4 * 4 + Q * (size_t)K * 4 + Q * kTopkCand * 8 + 256;
}

static inline char *align256(char *p) { return (char *)(((uintptr_t)p + 255) & ~(uintptr_t)255); }

void topk_carve(TopkArgs &a, void *ws, int n_queries) {
    if (a.n_max <= kTopkLdsCap) return;
    const size_t Q = (size_t)n_queries;
    char *p = align256((char *)ws);
    a.hist = (uint32_t *)p;
    p += Q * kTopkBins * 4;
    a.counters = (uint32_t *)p;
    p += Q * 4 * 4;
    a.sel = (int32_t *)p;
    p += Q * (size_t)a.K * 4;
    a.cand_key = (uint32_t *)p;
    p += Q * kTopkCand * 4;
    a.cand_idx = (int32_t *)p;
}

hipError_t launch_topk(const TopkArgs &a0, hipStream_t stream) {
    const int Q = a0.B * a0.T;
    if (a0.n_max <= kTopkLdsCap) {
        hipLaunchKernelGGL(topk_lds_kernel, dim3(Q), dim3(kWG), 0, stream, a0);
        return hipGetLastError();
    }
    TopkArgs a = a0;
    a.chunk = 2048;
    const int n_chunks = (a.n_max + a.chunk - 1) / a.chunk;
    const size_t clear_n = (size_t)Q * (kTopkBins + 4);
    int clear_blocks = (int)((clear_n + kAuxThreads - 1) / kAuxThreads);
    clear_blocks = clear_blocks < 4096 ? clear_blocks : 4096;
    hipLaunchKernelGGL(topk_clear_kernel, dim3(clear_blocks), dim3(kAuxThreads), 0, stream, a, Q);
    hipLaunchKernelGGL(topk_hist_kernel, dim3(n_chunks, Q), dim3(kAuxThreads), 0, stream, a);
    hipLaunchKernelGGL(topk_thresh_kernel, dim3(Q), dim3(kAuxThreads), 0, stream, a);
    hipLaunchKernelGGL(topk_filter_kernel, dim3(n_chunks, Q), dim3(kAuxThreads), 0, stream, a);
    hipLaunchKernelGGL(topk_final_kernel, dim3(Q), dim3(kWG), 0, stream, a);
    return hipGetLastError();
}

}  // namespace csa
