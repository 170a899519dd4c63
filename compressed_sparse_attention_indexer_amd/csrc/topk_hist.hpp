// First-level key histogram of the multi-workgroup top-k, shared by the
// histogram kernel and the scorer (which builds it while writing scores).
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace csa {

enum : int { kCtrlDone = 0, kCtrlBin = 1, kCtrlAbove = 3, kCtrlCand = 4 };
constexpr uint32_t kNoBin = 0xFFFFFFFFu;

// Called by every workgroup that builds the histogram, before anything else:
// the first workgroup of each query zero-fills the filter's counters, so the
// filter (a later kernel) always starts from zero whatever the workspace held.
__device__ __forceinline__ void hist_begin(uint32_t *ctrl) {
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        ctrl[kCtrlAbove] = 0u;
        ctrl[kCtrlCand] = 0u;
    }
}

// Workgroup-cooperative (256 threads).  Adds the workgroup's LDS histogram
// `lh` to the query's global histogram; the last of the query's `n_wg`
// workgroups to finish finds the bin holding the K-th largest key (counting
// from the top bin down), stores it in ctrl[kCtrlBin] (kNoBin if the
// histogram does not add up to n, e.g. a workspace that was not clean), and
// zero-fills the histogram and the done counter for the next call.
__device__ __forceinline__ void hist_publish(const uint32_t *lh, uint32_t *gh, uint32_t *ctrl, int n, int K,
                                             int n_wg, int *s_flag, uint32_t *s_wsum) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __syncthreads();
    for (int i = tid; i < kTopkBins; i += 256) {
        const uint32_t c = lh[i];
        if (c) atomicAdd(&gh[i], c);
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) *s_flag = atomicAdd(&ctrl[kCtrlDone], 1u) == (uint32_t)n_wg - 1u;
    __syncthreads();
    if (!*s_flag) return;
    __threadfence();
    constexpr int kPer = kTopkBins / 256;
    uint32_t h[kPer];
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        h[i] = __hip_atomic_load(&gh[kPer * tid + i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s += h[i];
    }
    uint32_t suf = s;  // sum over this lane and the lanes above it
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_down(suf, o);
        if (lane + o < 64) suf += t;
    }
    if (lane == 0) s_wsum[wave] = suf;
    __syncthreads();
    const uint32_t total = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
    for (int w = wave + 1; w < 4; ++w) suf += s_wsum[w];
    const uint32_t above = suf - s;
    const uint32_t need = (uint32_t)K;
    if (total != (uint32_t)n) {
        if (tid == 0) ctrl[kCtrlBin] = kNoBin;
    } else if (above < need && need <= suf) {
        uint32_t acc = above;
        for (int i = kPer - 1; i >= 0; --i) {
            if (acc < need && need <= acc + h[i]) {
                ctrl[kCtrlBin] = (uint32_t)(kPer * tid + i);
                break;
            }
            acc += h[i];
        }
    }
    __syncthreads();
    for (int i = tid; i < kTopkBins; i += 256) gh[i] = 0u;
    if (tid == 0) ctrl[kCtrlDone] = 0u;
}

}  // namespace csa
