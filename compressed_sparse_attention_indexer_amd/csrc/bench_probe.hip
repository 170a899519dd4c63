// Measurement helper for the benchmark (not part of the CSA path): a plain
// streaming read of a device buffer, to measure the HBM read bandwidth this
// part reaches, against which the path's kernels are compared.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// Each thread reads kUnroll 16-byte vectors per round, grid-stride, with
// nontemporal loads; the XOR of everything read is folded per workgroup and
// stored, so the loads cannot be dropped.
constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4 *__restrict__ src, size_t n_vec,
                                                               uint32_t *__restrict__ sink) {
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * kThreads;
    size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < n_vec; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n_vec; i += stride) {
        const u32x4 v = src[i];
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    __shared__ uint32_t red[kThreads / 64];
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int w = 0; w < kThreads / 64; ++w) r ^= red[w];
        sink[blockIdx.x] = r;
    }
}

}  // namespace

// Enqueue one streaming read of `bytes` (a multiple of 16) at src on `stream`;
// sink holds `blocks` uint32 values.  Returns a hipError_t.
extern "C" int csa_bench_stream_read(const void *src, size_t bytes, uint32_t *sink, int blocks, void *stream) {
    if (!src || !sink || blocks < 1 || (bytes & 15) || ((uintptr_t)src & 15)) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream,
                       (const u32x4 *)src, bytes / 16, sink);
    return (int)hipGetLastError();
}
