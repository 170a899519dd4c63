// Key histograms of the multi-workgroup top-k, shared by the histogram
// kernel, the scorer (which builds them while writing scores) and the
// selection kernels.  No global atomics: every workgroup stores a window of
// its own histogram with plain stores, and the consumer merges the windows.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace csa {

constexpr uint32_t kNoBin = 0xFFFFFFFFu;

// LDS histogram add.  Scores often crowd into one bin, and same-address LDS
// atomics serialize lane by lane, so lanes that share the first active lane's
// bin are counted with one atomic; the other lanes add on their own.
__device__ __forceinline__ void lds_hist_add(uint32_t *h, uint32_t bin, bool valid) {
    const uint64_t act = __ballot(valid);
    if (!act) return;
    const int leader = __builtin_ctzll(act);
    const uint32_t lb = __builtin_amdgcn_readlane(bin, leader);
    const bool same = valid && bin == lb;
    const uint64_t m = __ballot(same);
    if (lane_id() == leader) atomicAdd(&h[lb], (uint32_t)__popcll(m));
    if (valid && !same) atomicAdd(&h[bin], 1u);
}

// Workgroup of 256 threads: store the window of its 4096-bin LDS histogram `lh`
// that ends at its highest non-empty bin M: cnt[t] = lh[M - (kTopkWin - 1) + t]
// (0 below bin 0), hdr = M (or -1 when empty).  Bins within kTopkWin of the
// global highest bin are then exactly known from all windows together.
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

// The same for a workgroup of 256 threads whose threads already know the
// highest bin they added (mb, -1 if none): no scan of the histogram.
__device__ __forceinline__ void hist_window_store_top(const uint32_t *lh, int mb, int32_t *hdr, uint32_t *cnt,
                                                      int *s_red) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mb = max(mb, __shfl_xor(mb, o));
    if (lane == 0) s_red[wave] = mb;
    __syncthreads();  // also: every add to lh is done
    const int M = max(max(s_red[0], s_red[1]), max(s_red[2], s_red[3]));
    if (tid < kTopkWin) {
        const int b = M - (kTopkWin - 1) + tid;
        cnt[tid] = (M >= 0 && b >= 0) ? lh[b] : 0u;
    }
    if (tid == 0) *hdr = M;
}

// Merge n_win windows (hdr[w], cnt[w][kTopkWin]) into the exact histogram of
// the top kTopkWin bins below the global highest bin M, and return the bin
// holding the K-th largest key (kNoBin if it lies below that range or there is
// nothing).  Any block size that is a multiple of 64 (up to 1024); s_hist
// needs kTopkWin words, s_red one int per wave.  Four threads take a window
// (kTopkWin / 4 counts each).  Every header and the counts of the first blockDim/4
// windows are loaded in one round (the caller may have its own loads in
// flight too); further windows, if any, take one more round per blockDim/4.
__device__ __forceinline__ uint32_t window_threshold(const int32_t *hdr, const uint32_t *cnt, int n_win, int K,
                                                     int *s_red, uint32_t *s_hist) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nt = blockDim.x, nwaves = nt >> 6, per_pass = nt >> 2;
    const int seg = tid & 3;
    constexpr int kPerSeg = kTopkWin / 4;  // counts per thread of a window
    constexpr int kVecs = kPerSeg / 4;
    int mw = -1;
    u32x4_t x[kVecs];
    auto load_window = [&](int w) {
        mw = -1;
        if (w < n_win) {
            mw = hdr[w];
            const u32x4_t *src = (const u32x4_t *)(cnt + (size_t)w * kTopkWin + kPerSeg * seg);
#pragma unroll
            for (int i = 0; i < kVecs; ++i) x[i] = src[i];
        }
    };
    load_window(tid >> 2);  // issued before the header maximum below waits for its loads
    int m = -1;
    for (int w = tid; w < n_win; w += nt) m = max(m, hdr[w]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = max(m, __shfl_xor(m, o));
    if (lane == 0) s_red[wave] = m;
    for (int i = tid; i < kTopkWin; i += nt) s_hist[i] = 0u;
    __syncthreads();
    int M = -1;
    for (int w = 0; w < nwaves; ++w) M = max(M, s_red[w]);
    if (M < 0) return kNoBin;  // the same in every thread
    for (int w0 = 0;;) {
        if (mw >= 0) {
            const int off = mw - M + kPerSeg * seg;  // merged-window bin of this thread's first count
#pragma unroll
            for (int i = 0; i < kVecs; ++i)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int b = off + 4 * i + c;
                    if (x[i][c] && b >= 0 && b < kTopkWin) atomicAdd(&s_hist[b], x[i][c]);
                }
        }
        w0 += per_pass;
        if (w0 >= n_win) break;
        load_window(w0 + (tid >> 2));
    }
    __syncthreads();
    if (tid == 0) {
        uint32_t result = kNoBin, acc = 0;
        for (int t = kTopkWin - 1; t >= 0; --t) {
            acc += s_hist[t];
            if (acc >= (uint32_t)K) {
                const int b = M - (kTopkWin - 1) + t;
                result = b >= 0 ? (uint32_t)b : kNoBin;
                break;
            }
        }
        s_red[0] = (int)result;
    }
    __syncthreads();
    const uint32_t result = (uint32_t)s_red[0];
    __syncthreads();
    return result;
}

}  // namespace csa
