// KV / index-key compressor ("DeepSeek-V4 Architecture Analysis", INNOVATIONS
// 1: learned projection wkv and gating wgate, absolute position embeddings
// within each compression window, RMSNorm on the compressed output, RoPE on
// the rope dims; 4:1 with overlapping windows, 128:1; the indexer's own
// compressor adds a Hadamard rotation; "DeepSeek-V4-Flash" config table:
// compress_rope_theta, rms_norm_eps).
//
// Two launches.  (1) The projections of every supplied token, P = x [Wkv;
// Wgate]^T (bf16 in, fp32 out, v_mfma_f32_16x16x32_bf16), in one of two forms:
//   * few tokens (a decode step's window, an HCA window): weight streaming.  A
//     workgroup owns 16 output columns and all of hidden; its 8 waves split
//     hidden, each keeps its weight fragments in registers and sweeps the
//     token tiles, and the waves' sums meet in LDS.  Every weight byte is read
//     once, with a whole batch of loads in flight per wave.
//   * many tokens (a prefill chunk): a 128 x 128 LDS-tiled GEMM, 64 of hidden
//     per stage, double-buffered LDS fed from a 2-stage ring of register
//     prefetches, 8 waves of 64 x 32; hidden is split over 2-8
//     workgroups when the tiles alone would leave CUs idle, each split writing
//     its own fp32 partial.
// (2) One workgroup per compressed entry: token groups run an online softmax
// over their share of the window (gate logit + slot position embedding, per
// dim, the kv row weighted), the groups merge, then RMSNorm, RoPE on the rope
// slice (angle and its reduction modulo 2 pi in float64), optional normalized
// Hadamard rotation (fast Walsh-Hadamard transform across lanes), bf16 out.
#include "common.hpp"
#include "launch.hpp"

namespace csa {

namespace {
// weight-streaming projection
constexpr int kGvWaves = 8;
constexpr int kGvMaxTokens = 128;                     // 8 token tiles of 16
constexpr int kGvBatch = 8;                           // 64-wide hidden blocks per load batch
// tiled projection
constexpr int kGmTile = 128;                          // tokens and columns per workgroup tile
constexpr int kGmK = 64;                              // hidden per stage
constexpr int kGmRow = kGmK + 8;                      // LDS row pitch in bf16 (16 B pad)
constexpr int kGmStage = 2 * kGmTile * kGmRow;        // bf16 per stage (A then B)
constexpr int kGmMaxSplits = 8;
constexpr int kGmWaves = 8;                           // 2 x 4 waves of 64 x 32
// pooling
constexpr int kPoolThreads = 1024;
}  // namespace

// Weight row of projection column n: wkv rows first, then wgate rows.
__device__ __forceinline__ const uint16_t *proj_row(const CompressArgs &a, int n) {
    return n < a.out_dim ? (const uint16_t *)a.wkv + (size_t)n * a.hidden
                         : (const uint16_t *)a.wgate + (size_t)(n - a.out_dim) * a.hidden;
}

// MFMA operand layout used below: within a 64-wide hidden block, lane (e, g)
// (e = lane % 16, g = lane / 16) holds hidden [16 g, 16 g + 16) of row e as
// two 8-element halves, half j feeding k-step j.  Both operands use the same
// assignment, so each k-step pairs matching hidden indices and the two steps
// together cover the block once.
__global__ __launch_bounds__(64 * kGvWaves) void compress_gemv_kernel(CompressArgs a) {
    __shared__ float s_red[kGvWaves][256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = lane & 15, g = lane >> 4;
    const int N = 2 * a.out_dim;
    const int col0 = 16 * blockIdx.x;
    const int nblk = a.hidden / 64;
    const int n_mt = (a.tokens + 15) / 16;
    const uint16_t *wrow = proj_row(a, col0 + e) + 16 * g;
    f32x4_t acc[kGvMaxTokens / 16];
#pragma unroll
    for (int mt = 0; mt < kGvMaxTokens / 16; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // this wave's blocks: wave, wave + 8, ...; taken kGvBatch at a time, every load of a
    // batch issued before the first product (a batch past the end reloads the wave's last
    // block and drops its product)
    const int nb_w = (nblk - wave + kGvWaves - 1) / kGvWaves;
    for (int i0 = 0; i0 < nb_w; i0 += kGvBatch) {
        int off[kGvBatch];
        bf16x8_t w[kGvBatch][2];
#pragma unroll
        for (int i = 0; i < kGvBatch; ++i) {
            off[i] = 64 * (wave + kGvWaves * min(i0 + i, nb_w - 1));
            w[i][0] = *(const bf16x8_t *)(wrow + off[i]);
            w[i][1] = *(const bf16x8_t *)(wrow + off[i] + 8);
        }
#pragma unroll
        for (int mt = 0; mt < kGvMaxTokens / 16; ++mt) {
            if (mt >= n_mt) break;
            int t = 16 * mt + e;
            t = t < a.tokens ? t : a.tokens - 1;  // rows past the end repeat the last row; never stored
            const uint16_t *xrow = (const uint16_t *)a.x + (size_t)t * a.hidden + 16 * g;
            bf16x8_t xv[kGvBatch][2];
#pragma unroll
            for (int i = 0; i < kGvBatch; ++i) {
                xv[i][0] = *(const bf16x8_t *)(xrow + off[i]);
                xv[i][1] = *(const bf16x8_t *)(xrow + off[i] + 8);
            }
#pragma unroll
            for (int i = 0; i < kGvBatch; ++i) {
                if (i0 + i < nb_w) {
                    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv[i][0], w[i][0], acc[mt], 0, 0, 0);
                    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv[i][1], w[i][1], acc[mt], 0, 0, 0);
                }
            }
        }
    }
    // C layout: lane holds rows 4 g + r of the 16-token tile, column e
#pragma unroll
    for (int mt = 0; mt < kGvMaxTokens / 16; ++mt) {
        if (mt >= n_mt) break;
#pragma unroll
        for (int r = 0; r < 4; ++r) s_red[wave][16 * (4 * g + r) + e] = acc[mt][r];
        __syncthreads();
        if (threadIdx.x < 256) {
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < kGvWaves; ++w) v += s_red[w][threadIdx.x];
            const int t = 16 * mt + (threadIdx.x >> 4);
            if (t < a.tokens) a.part[(size_t)t * N + col0 + (threadIdx.x & 15)] = v;
        }
        __syncthreads();
    }
}

// P_s[t, n] = sum over split s's share of hidden of x[t, h] W[n, h].  Stage
// st's global loads are issued kAhead stages before its LDS copy (a ring of
// register slots); the LDS itself is double-buffered.  Tiles are numbered so
// that the column tiles of a token tile run on one XCD (consecutive workgroups
// go to consecutive XCDs) and share its x rows in that XCD's L2.  Measured on
// the 2,048-token chunk it is bound by how fast each CU's L1 is refilled (one
// 32 KiB stage per workgroup per 64 of hidden), not by the MFMA rate.
template <int kWaves, int kAhead>
__global__ __launch_bounds__(64 * kWaves) void compress_gemm_kernel(CompressArgs a) {
    constexpr int kThreads = 64 * kWaves;
    constexpr int kPass = kGmTile * 8 / kThreads;  // copy passes per operand tile (8 threads per 128-B row)
    constexpr int kWn = kWaves / 2;                 // waves along the columns (2 along the tokens)
    constexpr int kNt = kGmTile / kWn / 16;         // 16-column MFMA tiles per wave
    __shared__ uint16_t s_tile[2 * kGmStage];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int e = lane & 15, g = lane >> 4;
    const int wm = wave & 1, wn = wave >> 1;  // wave tile: 64 tokens x 16 kNt columns
    const int N = 2 * a.out_dim;
    const int n_m = gridDim.x, n_n = gridDim.y, n_tiles = n_m * n_n * gridDim.z;
    const int lin = blockIdx.x + n_m * (blockIdx.y + n_n * blockIdx.z);
    int tile = lin;
    if (n_tiles % 8 == 0) tile = (lin % 8) * (n_tiles / 8) + lin / 8;
    const int tn = tile % n_n, tm = (tile / n_n) % n_m, split = tile / (n_n * n_m);
    const int m0 = tm * kGmTile, n0 = tn * kGmTile;
    const int kspan = a.hidden / gridDim.z, kbeg = split * kspan;
    const int nst = kspan / kGmK;
    // global -> LDS copy: thread covers 16 B chunk (tid % 8) of rows tid / 8 + (kThreads / 8) p
    constexpr int kRowStep = kThreads / 8;
    const int cr = tid >> 3, cc = 8 * (tid & 7);
    const uint16_t *asrc[kPass], *bsrc[kPass];
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
        int t = m0 + cr + kRowStep * p;
        t = t < a.tokens ? t : a.tokens - 1;  // rows past the end repeat the last row; never stored
        asrc[p] = (const uint16_t *)a.x + (size_t)t * a.hidden + kbeg + cc;
        bsrc[p] = proj_row(a, n0 + cr + kRowStep * p) + kbeg + cc;
    }
    bf16x8_t ra[kAhead][kPass], rb[kAhead][kPass];
#define GM_FETCH(slot, st)                                                      \
    _Pragma("unroll") for (int p = 0; p < kPass; ++p) {                         \
        ra[slot][p] = *(const bf16x8_t *)(asrc[p] + (st) * kGmK);               \
        rb[slot][p] = *(const bf16x8_t *)(bsrc[p] + (st) * kGmK);               \
    }
#define GM_STASH(slot, buf)                                                     \
    {                                                                           \
        uint16_t *sa_ = s_tile + (buf) * kGmStage, *sb_ = sa_ + kGmTile * kGmRow; \
        _Pragma("unroll") for (int p = 0; p < kPass; ++p) {                     \
            *(bf16x8_t *)(sa_ + (cr + kRowStep * p) * kGmRow + cc) = ra[slot][p]; \
            *(bf16x8_t *)(sb_ + (cr + kRowStep * p) * kGmRow + cc) = rb[slot][p]; \
        }                                                                       \
    }
    f32x4_t acc[4][kNt];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < kNt; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // the loop body has no branches, so the compiler's memory counters wait only for the
    // slot being copied: stages past the end are fetched again from the last stage (in
    // bounds, never used), and kAhead divides the stage count
#pragma unroll
    for (int j = 0; j < kAhead; ++j) GM_FETCH(j, min(j, nst - 1))
    GM_STASH(0, 0)
    __syncthreads();
    for (int st0 = 0; st0 < nst; st0 += kAhead) {
#pragma unroll
        for (int j = 0; j < kAhead; ++j) {
            const int st = st0 + j;
            // slot j held stage st (already in LDS): refill it with stage st + kAhead
            GM_FETCH(j, min(st + kAhead, nst - 1))
            const uint16_t *sa = s_tile + (st & 1) * kGmStage, *sb = sa + kGmTile * kGmRow;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8_t af[4], bfr[kNt];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    af[i] = *(const bf16x8_t *)(sa + (64 * wm + 16 * i + e) * kGmRow + 16 * g + 8 * ks);
#pragma unroll
                for (int q = 0; q < kNt; ++q)
                    bfr[q] = *(const bf16x8_t *)(sb + (16 * kNt * wn + 16 * q + e) * kGmRow + 16 * g + 8 * ks);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int q = 0; q < kNt; ++q)
                        acc[i][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[q], acc[i][q], 0, 0, 0);
            }
            GM_STASH((j + 1) % kAhead, (st + 1) & 1)  // after the last stage: a copy nobody reads
            __syncthreads();
        }
    }
#undef GM_FETCH
#undef GM_STASH
    float *P = a.part + (size_t)split * a.tokens * N;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = m0 + 64 * wm + 16 * i + 4 * g + r;
            if (t >= a.tokens) continue;
#pragma unroll
            for (int q = 0; q < kNt; ++q) P[(size_t)t * N + n0 + 16 * kNt * wn + 16 * q + e] = acc[i][q][r];
        }
}

// RoPE factors of pair k of the rope slice at position pos: the angle
// pos * theta^(-2k / rope_dims) in float64 (positions reach 2^22), reduced
// modulo 2 pi in float64 (two-part constant), then a float sincos.
__device__ __forceinline__ void rope_factors(double pos, int k, int rope_dims, double ln_theta, float &cs, float &sn) {
    const double ang = pos * exp(-2.0 * k / rope_dims * ln_theta);
    const double n = rint(ang * 0.15915494309189535);
    double r = fma(-n, 6.283185307179586, ang);
    r = fma(-n, 2.4492935982947064e-16, r);
    sincosf((float)r, &sn, &cs);
}

// One workgroup per entry.  Thread (group, c) owns dims 4c .. 4c + 3 of token
// group `group`, which takes the window's tokens group, group + G, ...; group 0
// then merges the groups and finishes the entry, while another group works out
// the RoPE factors.
__global__ __launch_bounds__(kPoolThreads) void compress_pool_kernel(CompressArgs a) {
    __shared__ float s_m[kPoolThreads * 4], s_z[kPoolThreads * 4], s_s[kPoolThreads * 4];
    __shared__ float s_rope[2][256];
    __shared__ float s_red[16];
    const int D = a.out_dim, N = 2 * D, GS = D / 4, G = blockDim.x / GS;
    const int c = threadIdx.x % GS, grp = threadIdx.x / GS;
    const bool fin = grp == 0;
    const long ent = a.first_entry + blockIdx.x;
    const long last = (long)a.ratio * ent + a.ratio - 1, start = last - a.window + 1;
    const size_t split_stride = (size_t)a.tokens * N;
    f32x4_t gm = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (fin) gm = *(const f32x4_t *)(a.gamma + 4 * c);
    float m[4], z[4], s[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) m[k] = -INFINITY, z[k] = 0.f, s[k] = 0.f;
#pragma unroll 4
    for (long t = (start < 0 ? 0 : start) + grp; t <= last; t += G) {
        const float *row = a.part + (size_t)(t - a.pos0) * N + 4 * c;
        f32x4_t kv = *(const f32x4_t *)row, gt = *(const f32x4_t *)(row + D);
        for (int sp = 1; sp < a.n_splits; ++sp) {
            kv += *(const f32x4_t *)(row + sp * split_stride);
            gt += *(const f32x4_t *)(row + sp * split_stride + D);
        }
        gt += *(const f32x4_t *)(a.ape + (size_t)(t - start) * D + 4 * c);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float mn = fmaxf(m[k], gt[k]);
            const float sc = __expf(m[k] - mn), p = __expf(gt[k] - mn);
            z[k] = z[k] * sc + p;
            s[k] = s[k] * sc + p * kv[k];
            m[k] = mn;
        }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        s_m[4 * threadIdx.x + k] = m[k];
        s_z[4 * threadIdx.x + k] = z[k];
        s_s[4 * threadIdx.x + k] = s[k];
    }
    __syncthreads();
    const int r0 = D - a.rope_dims;
    if (grp == (G > 1 ? 1 : 0)) {  // RoPE factors of this thread's two pairs, for group 0
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int d = 4 * c + 2 * h;
            float cs = 1.f, sn = 0.f;
            if (d >= r0) rope_factors((double)(a.ratio * ent), (d - r0) / 2, a.rope_dims, a.rope_ln_theta, cs, sn);
            s_rope[0][2 * c + h] = cs;
            s_rope[1][2 * c + h] = sn;
        }
    }
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (fin) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float mm = -INFINITY;
            for (int q = 0; q < G; ++q) mm = fmaxf(mm, s_m[4 * (q * GS + c) + k]);
            float zz = 0.f, ss = 0.f;
            for (int q = 0; q < G; ++q) {
                const int i = 4 * (q * GS + c) + k;
                if (s_z[i] > 0.f) {  // a group that saw no token holds m = -inf, z = 0
                    const float w = __expf(s_m[i] - mm);
                    zz += s_z[i] * w;
                    ss += s_s[i] * w;
                }
            }
            v[k] = ss / zz;
        }
    }
    // RMSNorm over the D dims of group 0 (waves 0 .. nw - 1; other threads add 0)
    float sq = v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    sq = wave_sum(sq);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = (GS + 63) / 64;
    if (lane == 0) s_red[wave] = sq;
    __syncthreads();
    float tot = 0.f;
    for (int w = 0; w < nw; ++w) tot += s_red[w];
    const float inv = rsqrtf(tot / (float)D + a.rms_eps);
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = v[k] * inv * gm[k];
    // RoPE on the trailing rope_dims dims: pairs (4c, 4c + 1) and (4c + 2, 4c + 3)
    if (fin && 4 * c + 3 >= r0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float cs = s_rope[0][2 * c + h], sn = s_rope[1][2 * c + h];
            const float x0 = v[2 * h], x1 = v[2 * h + 1];
            v[2 * h] = x0 * cs - x1 * sn;
            v[2 * h + 1] = x0 * sn + x1 * cs;
        }
    }
    if (a.hadamard) {  // normalized Sylvester Hadamard rotation: one butterfly stage per bit of the dim index
        // bits 0 and 1: within the thread
        float u0 = v[0] + v[1], u1 = v[0] - v[1], u2 = v[2] + v[3], u3 = v[2] - v[3];
        v[0] = u0 + u2, v[2] = u0 - u2, v[1] = u1 + u3, v[3] = u1 - u3;
        // bits 2 .. : partner thread c ^ hl, a lane of the same wave while hl < 64
        for (int hl = 1; hl < GS && hl < 64; hl <<= 1) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float o = __shfl_xor(v[k], hl);
                v[k] = (c & hl) ? o - v[k] : v[k] + o;
            }
        }
        if (GS > 64) {  // out_dim 512: the last bit pairs the two waves of group 0, through LDS
            if (fin) {
#pragma unroll
                for (int k = 0; k < 4; ++k) s_z[4 * c + k] = v[k];
            }
            __syncthreads();
            if (fin) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float o = s_z[4 * (c ^ 64) + k];
                    v[k] = (c & 64) ? o - v[k] : v[k] + o;
                }
            }
        }
        const float sc = rsqrtf((float)D);
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] *= sc;
    }
    if (fin) {
        uint16_t *out = (uint16_t *)a.out + (size_t)blockIdx.x * D + 4 * c;
#pragma unroll
        for (int k = 0; k < 4; ++k) out[k] = __builtin_bit_cast(uint16_t, (__bf16)v[k]);
    }
}

int compress_splits(int tokens, int hidden, int out_dim) {
    if (tokens <= kGvMaxTokens) return 1;
    const int tiles = ((tokens + kGmTile - 1) / kGmTile) * ((2 * out_dim) / kGmTile);
    int s = 1;
    while (tiles * s < 256 && s < kGmMaxSplits && hidden % (2 * s * kGmK) == 0 && hidden / (2 * s) >= 4 * kGmK)
        s *= 2;
    return s;
}

hipError_t launch_compress(CompressArgs a, hipStream_t stream) {
    const int N = 2 * a.out_dim;
    if (a.tokens <= kGvMaxTokens) {
        hipLaunchKernelGGL(compress_gemv_kernel, dim3(N / 16), dim3(64 * kGvWaves), 0, stream, a);
    } else {
        const dim3 grid((a.tokens + kGmTile - 1) / kGmTile, N / kGmTile, a.n_splits);
        const int nst = a.hidden / a.n_splits / kGmK;  // stages of global loads in flight: 2 or 1
        constexpr int W = kGmWaves;
        if (nst % 2 == 0)
            hipLaunchKernelGGL((compress_gemm_kernel<W, 2>), grid, dim3(64 * W), 0, stream, a);
        else
            hipLaunchKernelGGL((compress_gemm_kernel<W, 1>), grid, dim3(64 * W), 0, stream, a);
    }
    const int gs = a.out_dim / 4;
    // token groups per entry: enough threads to cover one entry's window at decode; with many
    // entries the workgroups themselves fill the GPU, so small ones (all resident at once) do
    int groups = kPoolThreads / gs;
    while (groups > 1 && groups / 2 >= a.window) groups /= 2;  // no more groups than window tokens
    while (groups > 1 && (long)a.n_entries * groups * gs > 256L * 1024) groups /= 2;
    hipLaunchKernelGGL(compress_pool_kernel, dim3(a.n_entries), dim3(groups * gs), 0, stream, a);
    return hipGetLastError();
}

}  // namespace csa
