// Key histograms of the multi-workgroup top-k, shared by the histogram
// kernel, the scorer (which builds them while writing scores) and the
// selection kernels.  No global atomics: every workgroup stores a window of
// its own histogram with plain stores, and the consumer merges the windows.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace csa {

constexpr uint32_t kNoBin = 0xFFFFFFFFu;

// Block-wide exclusive scan for NT threads (a multiple of 64); s_wave holds
// NT / 64 ints.  Two barriers.
template <int NT>
__device__ __forceinline__ int block_scan_excl(int x, int *s_wave, int *total) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int inc = wave_incl_scan(x);
    if (lane == 63) s_wave[wave] = inc;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int c = s_wave[w];
        before += w < wave ? c : 0;
        all += c;
    }
    __syncthreads();
    *total = all;
    return before + inc - x;
}

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
    mb = wave_max_int(mb);
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
__device__ __forceinline__ int hist_window_store_top(const uint32_t *lh, int mb, int32_t *hdr, uint32_t *cnt,
                                                     int *s_red) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    mb = wave_max_int(mb);
    if (lane == 0) s_red[wave] = mb;
    __syncthreads();  // also: every add to lh is done
    const int M = max(max(s_red[0], s_red[1]), max(s_red[2], s_red[3]));
    if (tid < kTopkWin) {
        const int b = M - (kTopkWin - 1) + tid;
        cnt[tid] = (M >= 0 && b >= 0) ? lh[b] : 0u;
    }
    if (tid == 0) *hdr = M;
    return M;
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
    m = wave_max_int(m);
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
    if (tid < 64) {  // wave 0: the highest bin t whose count from the top reaches K
        const uint32_t c = lane < kTopkWin ? s_hist[lane] : 0u;
        const uint32_t inc = wave_incl_scan_u(c);
        const uint32_t suf = __builtin_amdgcn_readlane(inc, 63) - inc + c;  // bins t .. kTopkWin - 1
        const uint64_t reach = __ballot(lane < kTopkWin && suf >= (uint32_t)K);
        if (lane == 0) {
            uint32_t result = kNoBin;
            if (reach) {
                const int t = 63 - __builtin_clzll(reach);
                const int b = M - (kTopkWin - 1) + t;
                result = b >= 0 ? (uint32_t)b : kNoBin;
            }
            s_red[0] = (int)result;
        }
    }
    __syncthreads();
    const uint32_t result = (uint32_t)s_red[0];
    __syncthreads();
    return result;
}

// A scorer workgroup's entries for the selection (fused decode path): every
// entry of its stretch whose key bin is at or above `cut`, the lowest bin with
// at most `cap` entries at or above it.  lh is the stretch's kTopkBins-bin key
// histogram, keys[i] the key of entry first + i (i < n).  Writes hdr = {cut,
// count} and the emitted keys and indices in index order, keys past the count
// zeroed.  The selection can
// use the lists when every region's cut lies at or below the threshold bin:
// then each holds all of its region's entries at or above the threshold.
// NT threads (a multiple of 64 dividing kTopkBins); s_wave NT / 64 ints.
template <int NT>
__device__ void emit_region(const uint32_t *lh, const uint32_t *keys, int n, int first, int cap, int top,
                            int32_t *hdr, uint32_t *okey, int32_t *oidx, int *s_wave, int *s_cut) {
    constexpr int kPer = kTopkBins / NT;
    constexpr int kE = 8;  // consecutive entries per thread and round of the compaction
    const int tid = threadIdx.x, lane = tid & 63;
    // The cut from the 64 bins at and below the stretch's highest bin `top`
    // (wave 0, a DPP suffix sum): it lies there unless those bins hold no more
    // than cap entries while the stretch holds more, and then the block scan
    // over all the bins below decides.  A top bin holding more than cap alone
    // gives cut = top + 1: nothing is emitted, and the selection, seeing the
    // region's cut above its threshold bin or not, stays exact.
    if (tid < 64) {
        int cf = -2;  // -2: not decided here
        if (n <= cap) {
            cf = 0;
        } else if (top >= 0) {
            const int b = top - 63 + lane;
            const uint32_t cb = b >= 0 ? lh[b] : 0u;
            const uint32_t inc = wave_incl_scan_u(cb);
            const uint32_t tw = __builtin_amdgcn_readlane(inc, 63);
            const uint32_t suf = tw - inc + cb;  // entries in bins b .. top
            if (tw > (uint32_t)cap) {
                const uint64_t fit = __ballot(suf <= (uint32_t)cap);  // lanes l0 .. 63
                cf = fit ? top - 63 + __builtin_ctzll(fit) : top + 1;
            }
        }
        if (lane == 0) *s_cut = cf;
    }
    __syncthreads();
    if (*s_cut == -2) {  // the same in every thread
        const int v = NT - 1 - tid;  // this thread's bins [kPer v, kPer v + kPer): thread 0 takes the top range
        uint32_t h[kPer];
        int c = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            h[i] = lh[kPer * v + i];
            c += (int)h[i];
        }
        int tot;
        const int above = block_scan_excl<NT>(c, s_wave, &tot);  // entries in the bins above this thread's range
        if (tot <= cap) {
            if (tid == 0) *s_cut = 0;
        } else if (above <= cap && above + c > cap) {  // the range where the count from the top passes cap
            int run = above, cut = kPer * v + kPer;
            for (int i = kPer - 1; i >= 0; --i) {
                run += (int)h[i];
                if (run > cap) break;
                cut = kPer * v + i;
            }
            *s_cut = cut;
        }
        __syncthreads();
    }
    const uint32_t cut = (uint32_t)*s_cut;
    int written = 0;
    for (int i0 = 0; i0 < n; i0 += NT * kE) {
        uint32_t k[kE];
        int m = 0;
#pragma unroll
        for (int e = 0; e < kE; ++e) {
            const int i = i0 + kE * tid + e;
            k[e] = i < n ? keys[i] : 0u;
            m += i < n && (k[e] >> 20) >= cut;
        }
        int rt;
        int pos = written + block_scan_excl<NT>(m, s_wave, &rt);
#pragma unroll
        for (int e = 0; e < kE; ++e) {
            const int i = i0 + kE * tid + e;
            if (i < n && (k[e] >> 20) >= cut) {
                if (pos < cap) {
                    okey[pos] = k[e];
                    oidx[pos] = first + i;
                }
                ++pos;
            }
        }
        written += rt;
    }
    // the slots past the count read as key 0 (no real key is 0), so the
    // selection can tell used slots without the count
    for (int i = written + tid; i < cap; i += NT) okey[i] = 0u;
    if (tid == 0) {
        hdr[0] = (int32_t)cut;
        hdr[1] = written;  // at most cap by the choice of cut
    }
}

}  // namespace csa
