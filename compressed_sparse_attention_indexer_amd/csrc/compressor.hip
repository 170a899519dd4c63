// KV / index-key compressor ("DeepSeek-V4 Architecture Analysis", INNOVATIONS
// 1: learned projection wkv and gating wgate, absolute position embeddings
// within each compression window, RMSNorm on the compressed output, RoPE on
// the rope dims; 4:1 with overlapping windows, 128:1; the indexer's own
// compressor adds a Hadamard rotation; "DeepSeek-V4-Flash" config table:
// compress_rope_theta, rms_norm_eps).
//
// Two kernels.  (1) The projections of every supplied token, P = x [Wkv;
// Wgate]^T (bf16 in, fp32 out), on v_mfma_f32_16x16x32_bf16: a wave computes
// 32 tokens x 64 output columns, its A and B fragments read straight from
// global memory (L2 serves the repeats); the K dimension (hidden) is split
// over several workgroups when few tokens would leave the GPU idle (decode),
// each split writing its own fp32 partial.  (2) One workgroup per compressed
// entry, one thread per output-dim pair: sums the partials of the window's
// tokens, softmax over the tokens per dim (gate logits + the slot's position
// embedding), weighted kv sum, RMSNorm (block reduction), RoPE on the pairs
// of the rope slice (angle in float64: positions reach 2^20), optional
// normalized Hadamard rotation (in-LDS fast Walsh-Hadamard transform), bf16
// output.
#include "common.hpp"
#include "launch.hpp"

namespace csa {

namespace {
constexpr int kCpWaves = 4;
constexpr int kCpRows = 32;                     // tokens per workgroup tile
constexpr int kCpCols = 64 * kCpWaves;          // output columns per workgroup tile (64 per wave)
}  // namespace

// P_s[t, n] = sum_{h in split s} x[t, h] * W[n, h], W = [wkv; wgate] (n < 2*out_dim)
__global__ __launch_bounds__(64 * kCpWaves) void compress_project_kernel(CompressArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = lane & 15, g = lane >> 4;
    const int row0 = blockIdx.x * kCpRows;
    const int col0 = blockIdx.y * kCpCols + 64 * wave;
    const int split = blockIdx.z;
    const int N = 2 * a.out_dim;
    const int kspan = a.hidden / gridDim.z;
    const int k0 = split * kspan;
    const uint16_t *x = (const uint16_t *)a.x;
    // A fragments: token row0 + 16 mt + e; B fragments: column col0 + 16 nt + e
    const uint16_t *arow[2], *brow[4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        int t = row0 + 16 * mt + e;
        t = t < a.tokens ? t : a.tokens - 1;  // clamped rows compute garbage that is never stored
        arow[mt] = x + (size_t)t * a.hidden + k0 + 8 * g;
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int n = col0 + 16 * nt + e;
        const uint16_t *w = n < a.out_dim ? (const uint16_t *)a.wkv + (size_t)n * a.hidden
                                          : (const uint16_t *)a.wgate + (size_t)(n - a.out_dim) * a.hidden;
        brow[nt] = w + k0 + 8 * g;
    }
    f32x4_t acc[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < kspan; k += 32) {
        bf16x8_t af[2], bfr[4];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) af[mt] = *(const bf16x8_t *)(arow[mt] + k);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) bfr[nt] = *(const bf16x8_t *)(brow[nt] + k);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bfr[nt], acc[mt][nt], 0, 0, 0);
    }
    // C layout: lane holds rows 4g + r of the 16-row tile, column e
    float *P = a.part + (size_t)split * a.tokens * N;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = row0 + 16 * mt + 4 * g + r;
            if (t >= a.tokens) continue;
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) P[(size_t)t * N + col0 + 16 * nt + e] = acc[mt][nt][r];
        }
}

// One workgroup per entry; thread i owns output dims 2i and 2i + 1.
__global__ __launch_bounds__(256) void compress_pool_kernel(CompressArgs a) {
    __shared__ float s_red[4];
    __shared__ float s_v[512];
    const int i = threadIdx.x;  // blockDim.x = out_dim / 2
    const int lane = i & 63, wave = i >> 6, nwaves = (blockDim.x + 63) >> 6;
    const long ent = a.first_entry + blockIdx.x;
    const long last = (long)a.ratio * ent + a.ratio - 1, start = last - a.window + 1;
    const int N = 2 * a.out_dim, D = a.out_dim;
    const size_t split_stride = (size_t)a.tokens * N;
    float m[2] = {-INFINITY, -INFINITY}, z[2] = {0.f, 0.f}, s[2] = {0.f, 0.f};
    for (long t = start < 0 ? 0 : start; t <= last; ++t) {  // online softmax over the window's tokens
        const int slot = (int)(t - start);
        const float *row = a.part + (size_t)(t - a.pos0) * N;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int d = 2 * i + c;
            float kv = 0.f, gt = 0.f;
            for (int sp = 0; sp < a.n_splits; ++sp) {
                kv += row[sp * split_stride + d];
                gt += row[sp * split_stride + D + d];
            }
            gt += a.ape[(size_t)slot * D + d];
            const float mn = fmaxf(m[c], gt);
            const float sc = expf(m[c] - mn), p = expf(gt - mn);
            z[c] = z[c] * sc + p;
            s[c] = s[c] * sc + p * kv;
            m[c] = mn;
        }
    }
    float v[2] = {s[0] / z[0], s[1] / z[1]};
    // RMSNorm
    float ss = v[0] * v[0] + v[1] * v[1];
    ss = wave_sum(ss);
    if (lane == 0) s_red[wave] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int w = 0; w < nwaves; ++w) tot += s_red[w];
    const float inv = rsqrtf(tot / (float)D + a.rms_eps);
    v[0] = v[0] * inv * a.gamma[2 * i];
    v[1] = v[1] * inv * a.gamma[2 * i + 1];
    // RoPE on the trailing rope_dims dims: this thread's pair is pair k of that slice
    const int r0 = D - a.rope_dims;
    if (2 * i >= r0) {
        const int k = (2 * i - r0) / 2;
        const double ang = (double)(a.ratio * ent) * exp(-2.0 * k / a.rope_dims * log((double)a.rope_theta));
        double sn, cs;
        sincos(ang, &sn, &cs);
        const float x0 = v[0], x1 = v[1];
        v[0] = (float)(x0 * cs - x1 * sn);
        v[1] = (float)(x0 * sn + x1 * cs);
    }
    if (a.hadamard) {  // normalized Sylvester Hadamard rotation: in-place butterflies over LDS
        s_v[2 * i] = v[0];
        s_v[2 * i + 1] = v[1];
        for (int h = 1; h < D; h <<= 1) {
            __syncthreads();
            // each thread does one butterfly per stage: pair (p, p + h) with p having bit h clear
            const int p = ((i / h) * 2 * h) + (i % h);
            const float u = s_v[p], w = s_v[p + h];
            __syncthreads();
            s_v[p] = u + w;
            s_v[p + h] = u - w;
        }
        __syncthreads();
        const float sc = rsqrtf((float)D);
        v[0] = s_v[2 * i] * sc;
        v[1] = s_v[2 * i + 1] * sc;
    }
    uint16_t *out = (uint16_t *)a.out + (size_t)blockIdx.x * D + 2 * i;
    out[0] = __builtin_bit_cast(uint16_t, (__bf16)v[0]);
    out[1] = __builtin_bit_cast(uint16_t, (__bf16)v[1]);
}

int compress_splits(int tokens, int hidden, int out_dim) {
    const int tiles = ((tokens + kCpRows - 1) / kCpRows) * ((2 * out_dim) / kCpCols);
    int s = 1;
    while (tiles * s * 2 <= 512 && hidden % (64 * s) == 0 && hidden / (2 * s) >= 256) s *= 2;  // ~256+ workgroups
    return s;
}

hipError_t launch_compress(CompressArgs a, hipStream_t stream) {
    const dim3 g1((a.tokens + kCpRows - 1) / kCpRows, (2 * a.out_dim) / kCpCols, a.n_splits);
    hipLaunchKernelGGL(compress_project_kernel, g1, dim3(64 * kCpWaves), 0, stream, a);
    hipLaunchKernelGGL(compress_pool_kernel, dim3(a.n_entries), dim3(a.out_dim / 2), 0, stream, a);
    return hipGetLastError();
}

}  // namespace csa
