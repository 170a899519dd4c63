// Key histograms of the multi-workgroup top-k, shared by the histogram
// kernel, the scorer (which builds them while writing scores) and the
// selection kernels.  No global atomics: every workgroup stores a window of
// its own histogram with plain stores, and the consumer merges the windows.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace csa {

constexpr uint32_t kNoBin = 0xFFFFFFFFu;

// Wave-aggregated LDS histogram add: lanes holding the same bin are counted by
// one atomic (scores crowd into few bins, so per-lane atomics would serialize).
__device__ __forceinline__ void lds_hist_add(uint32_t *h, uint32_t bin, bool valid) {
    uint64_t rem = __ballot(valid);
    while (rem) {
        const int leader = __builtin_ctzll(rem);
        const uint32_t lb = __shfl(bin, leader);
        const uint64_t m = __ballot(valid && bin == lb) & rem;
        if (lane_id() == leader) atomicAdd(&h[lb], (uint32_t)__popcll(m));
        rem &= ~m;
    }
}

// Workgroup of 256 threads: store the window of its 4096-bin LDS histogram `lh`
// that ends at its highest non-empty bin M: cnt[t] = lh[M - 127 + t] (0 below
// bin 0), hdr = M (or -1 when empty).  Bins within 128 of the global highest
// bin are then exactly known from all windows together.
__device__ __forceinline__ void hist_window_store(const uint32_t *lh, int32_t *hdr, uint32_t *cnt, int *s_red) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __syncthreads();
    constexpr int kPer = kTopkBins / 256;
    int mb = -1;
#pragma unroll
    for (int i = kPer - 1; i >= 0; --i)
        if (mb < 0 && lh[kPer * tid + i]) mb = kPer * tid + i;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mb = max(mb, __shfl_xor(mb, o));
    if (lane == 0) s_red[wave] = mb;
    __syncthreads();
    const int M = max(max(s_red[0], s_red[1]), max(s_red[2], s_red[3]));
    if (tid < kTopkWin) {
        const int b = M - (kTopkWin - 1) + tid;
        cnt[tid] = (M >= 0 && b >= 0) ? lh[b] : 0u;
    }
    if (tid == 0) *hdr = M;
}

// Merge n_win windows (hdr[w], cnt[w][kTopkWin]) into the exact histogram of
// the top kTopkWin bins below the global highest bin, and return the bin that
// holds the K-th largest key (kNoBin if it lies below that range or there is
// nothing).  Any block size that is a multiple of 64 and >= kTopkWin.
__device__ __forceinline__ uint32_t window_threshold(const int32_t *hdr, const uint32_t *cnt, int n_win, int K,
                                                     int *s_red, uint32_t *s_bins) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nwaves = blockDim.x >> 6;
    int m = -1;
    for (int w = tid; w < n_win; w += blockDim.x) m = max(m, hdr[w]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = max(m, __shfl_xor(m, o));
    if (lane == 0) s_red[wave] = m;
    __syncthreads();
    int M = -1;
    for (int w = 0; w < nwaves; ++w) M = max(M, s_red[w]);
    __syncthreads();
    if (M < 0) return kNoBin;
    if (tid < kTopkWin) {
        const int b = M - (kTopkWin - 1) + tid;
        uint32_t c = 0;
        for (int w0 = 0; w0 < n_win; w0 += 8) {  // independent loads, 8 windows at a time
            uint32_t x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int w = w0 + u;
                const int mw = w < n_win ? hdr[w] : -1;
                const int off = b - (mw - (kTopkWin - 1));
                x[u] = (mw >= 0 && off >= 0 && off < kTopkWin) ? cnt[(size_t)w * kTopkWin + off] : 0u;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) c += x[u];
        }
        s_bins[tid] = c;
    }
    __syncthreads();
    uint32_t result = kNoBin;
    if (tid == 0) {
        uint32_t acc = 0;
        for (int t = kTopkWin - 1; t >= 0; --t) {
            acc += s_bins[t];
            const int b = M - (kTopkWin - 1) + t;
            if (acc >= (uint32_t)K) {
                result = b >= 0 ? (uint32_t)b : kNoBin;
                break;
            }
        }
        s_red[0] = (int)result;
    }
    __syncthreads();
    result = (uint32_t)s_red[0];
    __syncthreads();
    return result;
}

}  // namespace csa
