// Device helpers shared by the CSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Pointers read out of device pointer arrays are generic; loads through them
// compile to flat loads, which also count against the LDS wait counter.
// Reading through an explicit global (address space 1) pointer keeps them
// global loads, so LDS waits do not drain the memory pipeline.
template <typename T>
using gptr = const __attribute__((address_space(1))) T *;
template <typename T>
__device__ __forceinline__ gptr<T> as_global(const void *p) {
    return (gptr<T>)p;
}

// Number of compressed entries a query at raw position p sees: entry j covers
// raw tokens [r*j, r*j+r-1] and is visible iff r*j+r-1 <= p and j < L/r.
__device__ __forceinline__ int visible_entries(int64_t seq_len, int64_t pos, int ratio) {
    if (pos < 0 || seq_len <= 0) return 0;
    const int64_t n = seq_len / ratio;
    const int64_t v = (pos + 1) / ratio;
    return (int)(v < n ? v : n);
}

// Monotone map float -> uint32: a < b (as floats) <=> key(a) < key(b).
// -0.0 maps like +0.0 so equal floats give equal keys.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u << 1) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt() { return (1ull << lane_id()) - 1ull; }

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Window rows a query at p attends: raw positions [lo, hi], clamped to the
// window buffer [pos0, pos0 + rows - 1].  Returns the count (>= 0).
__device__ __forceinline__ int window_span(int pos, int window, int pos0, int rows, int *lo) {
    int a = pos - window + 1;
    a = a > 0 ? a : 0;
    a = a > pos0 ? a : pos0;
    int b = pos < pos0 + rows - 1 ? pos : pos0 + rows - 1;
    *lo = a;
    return b >= a ? b - a + 1 : 0;
}

}  // namespace csa
