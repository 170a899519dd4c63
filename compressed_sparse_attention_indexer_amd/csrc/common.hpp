// Device helpers shared by the CSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

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

// Cross-lane combines through the gfx950 lane swaps (VALU, no LDS round trip).
// swap16(a, b): lanes with bit 4 clear get (a of this lane, a of lane ^ 16)...
// precisely, per 32-lane half, v_permlane16_swap exchanges lanes 16..31 of its
// first operand with lanes 0..15 of its second, v_permlane32_swap lanes 32..63
// of the first with lanes 0..31 of the second.  pair16(a, b) returns, in every
// lane l, {x(l & ~16), x(l | 16)} where x is a for lanes with bit 4 clear and
// b for lanes with it set; pair32 the same over bit 5.  With a = b = v this is
// the pair {v(l & ~16), v(l | 16)}, the same ordered pair in both lanes.
struct LanePair {
    float lo, hi;
};
__device__ __forceinline__ LanePair pair16(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return LanePair{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ LanePair pair32(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return LanePair{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
// v(l) + v(l ^ 16) and v(l) + v(l ^ 32), bit-identical in both lanes of a pair
__device__ __forceinline__ float sum_xor16(float v) {
    const LanePair p = pair16(v, v);
    return p.lo + p.hi;
}
__device__ __forceinline__ float sum_xor32(float v) {
    const LanePair p = pair32(v, v);
    return p.lo + p.hi;
}
__device__ __forceinline__ float max_xor16(float v) {
    const LanePair p = pair16(v, v);
    return fmaxf(p.lo, p.hi);
}
__device__ __forceinline__ float max_xor32(float v) {
    const LanePair p = pair32(v, v);
    return fmaxf(p.lo, p.hi);
}

// Largest of v over the 16 lanes of each DPP row (lanes 16k .. 16k + 15), in
// every lane of the row: quad_perm [1,0,3,2] and [2,3,0,1] give each quad's
// maximum, row_half_mirror (lane i of 8 reads lane 7 - i) joins the two quads
// of a half row, row_mirror (lane i of 16 reads lane 15 - i) the two halves.
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)));
    return v;
}

// Inclusive prefix sum of x over the 64 lanes, on DPP: row_shr 1, 2, 4, 8
// within each 16-lane row (lanes shifted in from outside the row add 0), then
// row_bcast 15 (the last lane of rows 0 and 2 added to rows 1 and 3) and
// row_bcast 31 (lane 31 added to rows 2 and 3).  No LDS round trip, unlike a
// scan over __shfl_up.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);
    return x;
}

__device__ __forceinline__ uint32_t wave_incl_scan_u(uint32_t x) { return (uint32_t)wave_incl_scan((int)x); }

// Largest x over the 64 lanes, in every lane: the 16-lane row maximum on DPP
// (as row16_max), then across rows with the lane swaps.
__device__ __forceinline__ int wave_max_int(int x) {
    x = max(x, __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));
    x = max(x, __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));
    x = max(x, __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false));
    x = max(x, __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false));
    const auto a = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
    x = max((int)a[0], (int)a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
    return max((int)b[0], (int)b[1]);
}

// Sum of v over the 16 lanes of each DPP row, in every lane of the row (the
// pattern of row16_max; each step adds a lane pair in both orders, which give
// the same float, so every lane holds the same sum).
__device__ __forceinline__ float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));
    return v;
}

// Largest / sum of x over the 64 lanes, in every lane: DPP within the rows,
// then the lane swaps across them (no LDS round trip).
__device__ __forceinline__ float wave_max(float x) { return max_xor32(max_xor16(row16_max(x))); }

__device__ __forceinline__ float wave_sum(float x) { return sum_xor32(sum_xor16(row16_sum(x))); }

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
