// Multi-query attention over a row list with a per-head sink.
//
// Rows of one query: the selected compressed entries (top-k indices, or every
// visible entry for HCA), then the raw window rows of positions
// max(0, p-W+1)..p; key and value share one row unless separate values are
// given ("DeepSeek-V4 Architecture Analysis", INNOVATIONS 1: window, CSA/HCA
// compression, sink; INNOVATIONS 2: unified 512-d key/value).  One softmax
// over all rows plus the sink logit, which adds exp(sink) to the denominator
// and has no value vector.
#include "common.hpp"
#include "launch.hpp"

namespace csa {

namespace {

// Row i of a query's list -> key and value pointers (null if the row is not
// attended: padding index, out-of-range index, or past the list end).
struct RowList {
    int n_sel;   // rows taken from the compressed cache
    int n_rows;  // n_sel + window rows
    int wlo;     // first window position
    int n_ent;   // rows in the compressed cache of this sequence
};

__device__ __forceinline__ RowList make_rows(const MqaArgs &a, int qi) {
    const int b = qi / a.T;
    const int L = a.seq_len[b];
    const int p = a.q_pos[qi];
    RowList r;
    r.n_ent = L > 0 ? L / a.ratio : 0;
    const int nvis = visible_entries(L, p, a.ratio);
    r.n_sel = a.topk_idx ? a.K : nvis;
    const int nwin = window_span(p, a.W, a.win_pos0[b], a.win_rows[b], &r.wlo);
    r.n_rows = r.n_sel + nwin;
    return r;
}

// One sequence's cache bases (v / win_v null when key and value share a row).
template <typename T>
struct SeqRows {
    const T *kv, *v, *win, *win_v;
    int win_pos0;
};

template <typename T>
__device__ __forceinline__ SeqRows<T> seq_rows(const MqaArgs &a, int qi) {
    const int b = qi / a.T;
    return SeqRows<T>{(const T *)a.kv[b], a.v ? (const T *)a.v[b] : nullptr, (const T *)a.win[b],
                      a.win_v ? (const T *)a.win_v[b] : nullptr, a.win_pos0[b]};
}

// Key and value pointers of row i (null if the row is not attended), from the
// sequence's bases; `jl` is the row's list value when the caller has already
// read it (selected rows), else -2 to read it here.
template <typename T>
__device__ __forceinline__ void row_ptrs(const MqaArgs &a, const SeqRows<T> &sq, int qi, const RowList &rl, int i,
                                         const T **kp, const T **vp, int jl = -2) {
    *kp = nullptr;
    *vp = nullptr;
    if (i < 0 || i >= rl.n_rows) return;
    if (i < rl.n_sel) {
        const int j = !a.topk_idx ? i : jl != -2 ? jl : a.topk_idx[(size_t)qi * a.K + i];
        if (j < 0 || j >= rl.n_ent) return;
        *kp = sq.kv + (size_t)j * a.D;
        *vp = sq.v ? sq.v + (size_t)j * a.D : *kp;
    } else {
        const int pos = rl.wlo + (i - rl.n_sel);
        const size_t off = (size_t)(pos - sq.win_pos0) * a.D;
        *kp = sq.win + off;
        *vp = sq.win_v ? sq.win_v + off : *kp;
    }
}

template <typename T>
__device__ __forceinline__ void row_ptrs(const MqaArgs &a, int qi, const RowList &rl, int i, const T **kp,
                                         const T **vp) {
    row_ptrs(a, seq_rows<T>(a, qi), qi, rl, i, kp, vp);
}

}  // namespace

// ---------------------------------------------------------------------------
// fp32 VALU kernel (small shapes).  One workgroup per (head, query).  Pass 1
// finds the largest logit; pass 2 accumulates exp-weighted values 256 rows at
// a time (weights staged in LDS); the sink joins the max and the denominator.
__global__ __launch_bounds__(256) void mqa_f32_kernel(MqaArgs a) {
    extern __shared__ float smem[];
    float *sq = smem;                 // [D]
    float *sp = smem + a.D;           // [256] weights of the current row block
    __shared__ const float *svp[256];
    __shared__ float red[4];
    const int h = blockIdx.x, qi = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const RowList rl = make_rows(a, qi);
    const float *qrow = (const float *)a.q + ((size_t)qi * a.H + h) * a.D;
    for (int d = tid; d < a.D; d += 256) sq[d] = qrow[d];
    __syncthreads();
    auto logit = [&](const float *k) {
        float dot = 0.f;
        for (int d = 0; d < a.D; ++d) dot = fmaf(sq[d], k[d], dot);
        return dot * a.scale;
    };
    float m = -INFINITY;
    for (int i = tid; i < rl.n_rows; i += 256) {
        const float *kp, *vp;
        row_ptrs(a, qi, rl, i, &kp, &vp);
        if (kp) m = fmaxf(m, logit(kp));
    }
    m = wave_max(m);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float sink = a.sink[h];
    m = fmaxf(m, sink);
    __syncthreads();
    float l = 0.f;
    float acc0 = 0.f, acc1 = 0.f;  // d = tid and d = tid + 256
    for (int r0 = 0; r0 < rl.n_rows; r0 += 256) {
        const float *kp, *vp;
        row_ptrs(a, qi, rl, r0 + tid, &kp, &vp);
        const float pw = kp ? expf(logit(kp) - m) : 0.f;
        l += pw;
        sp[tid] = pw;
        svp[tid] = vp;
        __syncthreads();
        const int nb = rl.n_rows - r0 < 256 ? rl.n_rows - r0 : 256;
        for (int t = 0; t < nb; ++t) {
            const float *v = svp[t];
            if (!v) continue;
            if (tid < a.D) acc0 = fmaf(sp[t], v[tid], acc0);
            if (tid + 256 < a.D) acc1 = fmaf(sp[t], v[tid + 256], acc1);
        }
        __syncthreads();
    }
    l = wave_sum(l);
    if (lane == 0) red[wave] = l;
    __syncthreads();
    l = red[0] + red[1] + red[2] + red[3] + expf(sink - m);
    float *orow = a.out + ((size_t)qi * a.H + h) * a.D;
    if (tid < a.D) orow[tid] = acc0 / l;
    if (tid + 256 < a.D) orow[tid + 256] = acc1 / l;
    if (a.lse && tid == 0) a.lse[(size_t)qi * a.H + h] = m + logf(l);
}

// ---------------------------------------------------------------------------
// bf16 split-K MFMA kernel, D = 512, 16 * HG heads per workgroup (launched
// with HG = 2: 32 heads, so 64 heads take two workgroups and 128 heads four).
// Grid (splits, queries, Z head groups) while every workgroup of the launch is
// resident at once (two per CU): the Z workgroups of a (query, split) pair are
// then S Q ids apart, a multiple of 8 on the decode shapes, so they share an
// XCD (workgroups go to the 8 XCDs round-robin) and each row crosses into its
// L2 once.  Larger launches take a one-dimensional grid in which a pair's Z
// workgroups are 8 ids apart inside each run of 8 Z ids, so they are also
// dispatched together (with the head group as the slowest dimension the 4,096
// workgroups of a 2,048-query chunk fetched 1.47x their rows and queries, and
// the attention took 397 against 371 us); on the resident decode launches the
// one-dimensional order measured 0.2-0.8 us slower.  With 4-wave workgroups two of them share a
// CU (launch bounds ask for it: VGPRs stay at or below 256); their tiles'
// barrier phases (staging, QK, the logit exchange, softmax, PV) then overlap
// instead of running in lockstep, which took the decode step's attention from
// 10.8 to 8.7 us against one 8-wave workgroup of 64 heads per CU.
//
// Workgroup = one (query, split): 2*HG waves; wave (hg, dh) owns heads
// [16hg, 16hg+16) and output dims [256dh, 256dh+256).  Rows stream through
// LDS 32 at a time as bf16 rows [32][520] (padded), gathered with 16-byte
// loads (each thread one row, a prefetch one tile ahead in registers); a
// separate value row set gets its own buffer.
// QK: S^T[rows x heads] = K * Q^T on v_mfma_f32_16x16x32_bf16, each wave over
// its 256 dims; the two halves are summed through LDS (a + b in both waves,
// so both see bit-identical logits).  Online softmax in fp32 (log2 units).
// PV: O[heads x d] += P * V on v_mfma_f32_16x16x32_bf16.  P stays in
// registers exactly as QK left it (its row order defines the k order of V),
// split into a bf16 high part and a bf16 remainder (two MFMAs, about 16
// significant bits); the V fragments come straight from the row-major tile
// through gfx950's transposing LDS read (ds_read_b64_tr_b16), two per
// fragment.
// Output: partial (m, l, O) per split, or the final result with the sink when
// there is one split.
namespace {
constexpr int kD = 512;
constexpr int kTile = 32;
constexpr int kKrowStride = kD + 16;  // bf16 elements per staged row (1056 B: HCA 26.3 -> 25.8 us against 1040 B)
constexpr float kLazyMax = 8.f;       // log2 headroom of the running softmax reference
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));

// Transposing LDS read (gfx950): within each group of 16 lanes, lane i gets
// element i % 4 of the 8-byte vectors addressed by lanes i / 4, 4 + i / 4,
// 8 + i / 4 and 12 + i / 4 (in that order).  With lane s of the group
// addressing row r0 + s / 4, columns c0 + 4 (s % 4) .. + 3 of a row-major
// bf16 tile, lane i receives rows r0 .. r0 + 3 of column c0 + i.
__device__ __forceinline__ v4i16_t lds_read_tr16(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t *)p);
}
}  // namespace

template <int HG, bool kSepV>
__global__ __launch_bounds__(128 * HG, 2) void mqa_bf16_kernel(MqaArgs a) {
    constexpr int NW = 2 * HG;                // waves
    constexpr int RPW = kTile / NW;           // staged rows per wave
    constexpr int LPR = 64 / RPW;             // lanes per staged row
    constexpr int CPL = 64 / LPR;             // 16-byte chunks per lane
    static_assert(kTile % NW == 0 && 64 % RPW == 0, "staging layout");

    __shared__ __attribute__((aligned(16))) uint16_t krow[kTile * kKrowStride];
    __shared__ __attribute__((aligned(16))) uint16_t vrow_sep[kSepV ? kTile * kKrowStride : 8];  // separate values only
    __shared__ float xs[NW][8][64];
    __shared__ int rowok[kTile];

    const int Z = a.H / (16 * HG);  // head-group workgroups per (query, split), 2 or more
    int qi, split, zi;
    if (gridDim.z == 1) {  // one-dimensional grid
        const int pair = (int)blockIdx.x / (8 * Z) * 8 + (int)blockIdx.x % 8;
        if (pair >= a.n_splits * a.B * a.T) return;  // padding of the last run of 8 Z ids
        qi = pair / a.n_splits;
        split = pair % a.n_splits;
        zi = (int)blockIdx.x / 8 % Z;
    } else {
        qi = blockIdx.y;
        split = blockIdx.x;
        zi = blockIdx.z;
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int e = lane & 15, g = lane >> 4;
    const int hg = wave >> 1, dh = wave & 1;
    const int h_off = 16 * HG * zi;  // this workgroup's heads: h_off .. h_off + 16 HG - 1
    // q, the sequence's cache bases and the first tile's list value of this
    // thread's staging row are read in the same round as the query's row counts
    // (i < K is inside the top-k list whatever the counts; the row itself is
    // checked once they are known).
    // B fragments of Q^T: head 16hg + e, dims 256dh + 32ks + 8g .. +8.
    bf16x8_t qf[8];
    {
        const uint16_t *qrow = (const uint16_t *)a.q + ((size_t)qi * a.H + h_off + 16 * hg + e) * kD + 256 * dh + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qf[ks] = *(const bf16x8_t *)(qrow + 32 * ks);
    }
    const SeqRows<uint16_t> sq = seq_rows<uint16_t>(a, qi);
    const int srow0 = wave * RPW + lane / LPR;
    // this split's rows: whole tiles, the query's tiles dealt as evenly as possible over the splits
    const int r0 = (int)((long long)split * a.n_tiles / a.n_splits) * kTile;
    const int r_end = (int)((long long)(split + 1) * a.n_tiles / a.n_splits) * kTile;
    const int i_first = r0 + srow0;
    const int j_first = a.topk_idx && i_first < a.K ? a.topk_idx[(size_t)qi * a.K + i_first] : -2;
    const RowList rl = make_rows(a, qi);
    const int r1 = r_end < rl.n_rows ? r_end : rl.n_rows;
    const int ntiles = r1 > r0 ? (r1 - r0 + kTile - 1) / kTile : 0;
    const float scale2 = a.scale * kLog2e;

    f32x4_t o[16];
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;  // head 16hg + e, log2 units

    // staging role: one row, CPL chunks of 16 bytes
    // (a group of LPR consecutive lanes takes one row, 8 with HG = 2, so each
    // 8-lane phase of the 16-byte LDS writes covers 128 contiguous bytes)
    const int srow = wave * RPW + lane / LPR;
    const int cg = lane % LPR;
    u32x4_t kreg[CPL], vreg[kSepV ? CPL : 1];
    bool have_row = false;
    // a missing row (padding, out of range, past the list) reads this query's q
    // instead: finite values whose logit is masked to -inf, so its weight is 0
    const uint16_t *dummy = (const uint16_t *)a.q + (size_t)qi * a.H * kD;
    // top-k list value of this thread's staging row in tile t (-2 where the row
    // is not a selected entry), read one tile ahead of the row itself: read
    // inside the row fetch, each tile's row loads waited a whole global round
    // trip for their index first
    auto list_value = [&](int t) {
        const int i = r0 + t * kTile + srow;
        return a.topk_idx && i < r1 && i < rl.n_sel ? a.topk_idx[(size_t)qi * a.K + i] : -2;
    };
    auto fetch = [&](int t, int jl) {
        const uint16_t *kp, *vp;
        row_ptrs(a, sq, qi, rl, r0 + t * kTile + srow < r1 ? r0 + t * kTile + srow : -1, &kp, &vp, jl);
        have_row = kp != nullptr;
        if (!have_row) kp = vp = dummy;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int ch = cg + LPR * c;
            kreg[c] = *as_global<u32x4_t>(kp + 8 * ch);
            if (kSepV) vreg[c] = *as_global<u32x4_t>(vp + 8 * ch);
        }
    };
    int j_next = -2;  // list value for the next tile's fetch
    if (ntiles > 0) {
        fetch(0, j_first);
        if (ntiles > 1) j_next = list_value(1);
    }

    for (int t = 0; t < ntiles; ++t) {
        __syncthreads();  // previous tile fully consumed
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int ch = cg + LPR * c;
            *(u32x4_t *)&krow[srow * kKrowStride + 8 * ch] = kreg[c];
            if (kSepV) *(u32x4_t *)&vrow_sep[srow * kKrowStride + 8 * ch] = vreg[c];
        }
        if (cg == 0) rowok[srow] = have_row;
        if (t + 1 < ntiles) {
            fetch(t + 1, j_next);
            if (t + 2 < ntiles) j_next = list_value(t + 2);
        }
        __syncthreads();

        // QK over this wave's 256 dims: the two row tiles' chains interleaved,
        // the fragment reads kept eight ahead of the MFMAs (left to itself the
        // scheduler let each MFMA wait out the latency of the read just before it)
        f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
        bf16x8_t kf[8][2];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                kf[ks][mt] = *(const bf16x8_t *)&krow[(16 * mt + e) * kKrowStride + 256 * dh + 32 * ks + 8 * g];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks][mt], qf[ks], sacc[mt], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 8, 0);
#pragma unroll
        for (int v = 0; v < 8; ++v) xs[wave][v][lane] = sacc[v >> 2][v & 3];
        __syncthreads();
        float z[8];
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            const float s = sacc[v >> 2][v & 3] + xs[wave ^ 1][v][lane];
            const int row = 16 * (v >> 2) + 4 * g + (v & 3);
            z[v] = rowok[row] ? s * scale2 : -INFINITY;
        }
        // online softmax for head 16hg + e (rows spread over the 4 lane groups)
        float mx = z[0];
#pragma unroll
        for (int v = 1; v < 8; ++v) mx = fmaxf(mx, z[v]);
        mx = max_xor16(mx);
        mx = max_xor32(mx);
        // The reference max moves only when a logit passes it by more than kLazyMax (log2
        // units, also on the first finite logit): weights stay below 2^kLazyMax, and the
        // output accumulators are rescaled only when it moves.
        const bool move = mx > m_run + kLazyMax;
        const float m_ref = move ? mx : m_run;
        const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
        const float alpha = move ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.f;
        float pv[8], ls = 0.f;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            pv[v] = __builtin_amdgcn_exp2f(z[v] - m_use);
            ls += pv[v];
        }
        ls = sum_xor16(ls);
        ls = sum_xor32(ls);
        l_run = l_run * alpha + ls;
        m_run = m_ref;
        if (__any(move)) {
            float ar[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * g + r);
#pragma unroll
            for (int dt = 0; dt < 16; ++dt)
#pragma unroll
                for (int r = 0; r < 4; ++r) o[dt][r] *= ar[r];
        }
        bf16x8_t ph, pl;  // P = ph + pl, each part bf16
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            ph[v] = (__bf16)pv[v];
            pl[v] = (__bf16)(pv[v] - (float)ph[v]);
        }
        const uint16_t *vrow = kSepV ? vrow_sep : krow;
        const int s16 = lane & 15;  // this lane's address role in the transposing read
        // PV over this wave's 256 output dims, two dt at a time so consecutive
        // MFMAs are independent (each accumulator still takes its high part
        // before its remainder); the transposing reads kept eight ahead.
        bf16x8_t vf[16];
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) {
            // B fragment: V[rows 4g .. 4g+3 and 16+4g .. 16+4g+3][d = 256dh + 16dt + e]
            const uint16_t *vp0 = vrow + (4 * g + (s16 >> 2)) * kKrowStride + 256 * dh + 16 * dt + 4 * (s16 & 3);
            const v4i16_t lo = lds_read_tr16(vp0);
            const v4i16_t hi = lds_read_tr16(vp0 + 16 * kKrowStride);
            vf[dt] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int dt = 0; dt < 16; dt += 2) {
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vf[dt], o[dt], 0, 0, 0);
            o[dt + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vf[dt + 1], o[dt + 1], 0, 0, 0);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vf[dt], o[dt], 0, 0, 0);
            o[dt + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vf[dt + 1], o[dt + 1], 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
#pragma unroll
        for (int i = 0; i < 12; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 8, 0);
    }

    // epilogue: C layout holds O[head 16hg + 4g + r][d = 256dh + 16dt + e]
    const int hbase = h_off + 16 * hg + 4 * g;
    if (a.n_splits == 1) {
        const float sink2 = a.sink[h_off + 16 * hg + e] * kLog2e;
        const float M = fmaxf(m_run, sink2);
        const float lf = l_run * exp2f(m_run - M) + exp2f(sink2 - M);
        const float f = exp2f(m_run - M) / lf;
        float fr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) fr[r] = __shfl(f, 4 * g + r);
#pragma unroll
        for (int dt = 0; dt < 16; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                a.out[((size_t)qi * a.H + hbase + r) * kD + 256 * dh + 16 * dt + e] = o[dt][r] * fr[r];
        if (a.lse && dh == 0 && g == 0) a.lse[(size_t)qi * a.H + h_off + 16 * hg + e] = M * kLn2 + logf(lf);
    } else {
        // Partial of this split: (m, l) per head, and O / l in fp16 stored the
        // way the MFMA tiles lie in registers: the 16-byte vector at
        // [qi, split, head group, dh, dt pair p, lane] (head group = the
        // query's 16-head group h_off / 16 + hg, whatever HG is) holds heads
        // 16hg + 4g + r (r = 0..3) at dims 256dh + 16dt + e for dt = 2p and 2p + 1.
        // Each head's 256 values of this dim half are scaled by a power of two
        // that brings their largest magnitude into [2^14, 2^15), and the
        // inverse kept next to (m, l): any finite bf16 value range fits fp16's
        // 16 significant bits without overflow or subnormal loss.
        const size_t ps = (size_t)qi * a.n_splits + split;
        if (dh == 0 && g == 0) {
            a.part_ml[(ps * a.H + h_off + 16 * hg + e) * 4 + 0] = m_run;
            a.part_ml[(ps * a.H + h_off + 16 * hg + e) * 4 + 1] = l_run;
        }
        if (ntiles > 0) {
            const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
            float ir[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) ir[r] = __shfl(inv, 4 * g + r);
#pragma unroll
            for (int r = 0; r < 4; ++r) {  // head 16hg + 4g + r: largest |O/l| over its 256 dims here
                float mx = 0.f;
#pragma unroll
                for (int dt = 0; dt < 16; ++dt) mx = fmaxf(mx, fabsf(o[dt][r]));
                mx = row16_max(mx) * ir[r];  // over the 16 lanes e
                // 2^k with k = 14 - floor(log2(mx)) (mx = f 2^x with f in [0.5, 1)),
                // kept within fp32's normal range
                int k = mx > 0.f ? 15 - __builtin_amdgcn_frexp_expf(mx) : 0;
                k = k < -100 ? -100 : (k > 100 ? 100 : k);
                ir[r] *= ldexpf(1.f, k);
                if (e == 0) a.part_ml[(ps * a.H + h_off + 16 * hg + 4 * g + r) * 4 + 2 + dh] = ldexpf(1.f, -k);
            }
            u32x4_t *dst = (u32x4_t *)a.part_o + ((ps * Z + zi) * NW + wave) * 8 * 64 + lane;
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                uint32_t w4[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {  // word k: dt = 2p + k/2, heads r = 2(k%2), 2(k%2) + 1
                    const int dt = 2 * p + (k >> 1), r = 2 * (k & 1);
                    const _Float16 lo = (_Float16)(o[dt][r] * ir[r]);
                    const _Float16 hi = (_Float16)(o[dt][r + 1] * ir[r + 1]);
                    w4[k] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
                }
                dst[p * 64] = u32x4_t{w4[0], w4[1], w4[2], w4[3]};
            }
        }
    }
}

// Merge split partials with the sink, counted once (H = 64 or 128).
// Workgroup = (16-head group hg, lane group g, dim part dq of Zq, query):
// heads h0 .. h0 + 3 (h0 = 16hg + 4g) at 512 / Zq of the dims (Zq = 1, 2, 4 or 8,
// chosen so the launch has about 256 workgroups, 512 with many splits).  A 16-byte partial vector
// holds those 4 heads at two dims; the part's 256 / Zq vector positions of a
// split are spread over 256 / Zq threads (position: half dh, dt pair p,
// column e), and thread group sg of Zq folds splits sg, sg + Zq, ... , so with
// few queries every CU in the launch streams only a part of a head group's
// partials.  Wave r first turns head
// h0 + r's (m, l) pairs into per-split weights and the total (lanes over the
// splits; wave max and sum), into LDS, while the first partial vectors are
// already in flight; then each thread group folds its splits (the next
// batch's loads issued before the current batch is used), and the groups'
// sums meet in LDS.  Splits without rows (l = 0) get weight 0; their vectors (never
// written) are not used.
constexpr int kCombineMaxSplits = 1024;
template <int Zq>
__global__ __launch_bounds__(256) void mqa_combine_kernel(MqaArgs a) {
    constexpr int kBatch = 16;
    __shared__ float s_w[kCombineMaxSplits][4][2];  // split weight times the partial's scale, per dim half
    __shared__ float s_M[4], s_L[4];
    __shared__ float s_acc[1792];  // (Zq - 1) groups x 8 sums x 256 / Zq positions
    const int qi = blockIdx.y, dq = blockIdx.z;
    const int hg = blockIdx.x >> 2, g = blockIdx.x & 3;
    const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63;
    constexpr int npos = 256 / Zq;
    const int sg = tid / npos, c = tid % npos;
    const int pos = dq * npos + c;  // 0 .. 255 over the head group's 512 dims
    const int dh = pos >> 7, p = (pos >> 4) & 7, e = pos & 15;
    const int lane = 16 * g + e;
    const int h0 = 16 * hg + 4 * g;
    const int S = a.n_splits;
    // partial vectors: [qi, split, 16-head group hg, dh, dt pair, lane], here
    // indexed as 64-head block z = hg / 4 and (hg % 4, dh) inside it
    const int Z = a.H / 64, z = hg >> 2, wave_l = 2 * (hg & 3) + dh;
    const u32x4_t *src = (const u32x4_t *)a.part_o + ((((size_t)qi * S * Z + z) * 8 + wave_l) * 8 + p) * 64 + lane;
    const size_t sstride = (size_t)Z * 8 * 8 * 64;  // vectors per split
    // this thread group's splits: sg, sg + Zq, ...: n_mine of them
    const int n_mine = S > sg ? (S - sg + Zq - 1) / Zq : 0;
    u32x4_t ov[2][kBatch];
    auto load_batch = [&](u32x4_t (&v)[kBatch], int i0) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = i0 + u < n_mine ? i0 + u : n_mine - 1;  // clamped: in bounds, unconditional
            v[u] = src[(size_t)(sg + Zq * i) * sstride];
        }
    };
    if (n_mine > 0) load_batch(ov[0], 0);
    {  // weights of head h0 + wv; the first 64 splits' (m, l) pairs stay in registers
        const float sink2 = a.sink[h0 + wv] * kLog2e;
        float4 ml0 = float4{0.f, 0.f, 0.f, 0.f};  // m, l, inverse scales of the two dim halves
        if (ln < S) ml0 = *(const float4 *)(a.part_ml + (((size_t)qi * S + ln) * a.H + h0 + wv) * 4);
        float M = ml0.y > 0.f ? fmaxf(sink2, ml0.x) : sink2;
        for (int s = ln + 64; s < S; s += 64) {
            const float *ml = a.part_ml + (((size_t)qi * S + s) * a.H + h0 + wv) * 4;
            if (ml[1] > 0.f) M = fmaxf(M, ml[0]);
        }
        M = wave_max(M);
        float L = 0.f;
        if (ln < S) {
            const float w = ml0.y > 0.f ? ml0.y * exp2f(ml0.x - M) : 0.f;
            s_w[ln][wv][0] = w > 0.f ? w * ml0.z : 0.f;  // a split without rows never wrote its scales
            s_w[ln][wv][1] = w > 0.f ? w * ml0.w : 0.f;
            L += w;
        }
        for (int s = ln + 64; s < S; s += 64) {
            const float *ml = a.part_ml + (((size_t)qi * S + s) * a.H + h0 + wv) * 4;
            const float l = ml[1];
            const float w = l > 0.f ? l * exp2f(ml[0] - M) : 0.f;
            s_w[s][wv][0] = w > 0.f ? w * ml[2] : 0.f;
            s_w[s][wv][1] = w > 0.f ? w * ml[3] : 0.f;
            L += w;
        }
        L = wave_sum(L);
        if (ln == 0) {
            s_M[wv] = M;
            s_L[wv] = L + (sink2 > -INFINITY ? exp2f(sink2 - M) : 0.f);
        }
    }
    __syncthreads();
    float acc[4][2] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
    auto fold = [&](const u32x4_t (&v)[kBatch], int i0) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (i0 + u >= n_mine) break;
            const int s = sg + Zq * (i0 + u);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float w = s_w[s][r][dh];
                if (w == 0.f) continue;  // also keeps unwritten partials out
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {  // dt = 2p + kk: word 2kk + r/2, half r%2
                    const uint32_t wd = v[u][2 * kk + (r >> 1)];
                    const uint16_t hb = (uint16_t)((r & 1) ? (wd >> 16) : (wd & 0xFFFFu));
                    acc[r][kk] = fmaf(w, (float)__builtin_bit_cast(_Float16, hb), acc[r][kk]);
                }
            }
        }
    };
    for (int i0 = 0; i0 < n_mine; i0 += 2 * kBatch) {
        if (i0 + kBatch < n_mine) load_batch(ov[1], i0 + kBatch);
        fold(ov[0], i0);
        if (i0 + kBatch >= n_mine) break;
        if (i0 + 2 * kBatch < n_mine) load_batch(ov[0], i0 + 2 * kBatch);
        fold(ov[1], i0 + kBatch);
    }
    // the groups' sums meet in group 0
    if (sg > 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) s_acc[((sg - 1) * 8 + 2 * r + kk) * npos + c] = acc[r][kk];
    }
    __syncthreads();
    if (sg != 0) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float L = s_L[r];
        const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            float v = acc[r][kk];
            for (int q = 1; q < Zq; ++q) v += s_acc[((q - 1) * 8 + 2 * r + kk) * npos + c];
            a.out[((size_t)qi * a.H + h0 + r) * kD + 256 * dh + 16 * (2 * p + kk) + e] = v * inv;
        }
        if (a.lse && dq == 0 && tid == 0) a.lse[(size_t)qi * a.H + h0 + r] = s_M[r] * kLn2 + logf(L);
    }
}

constexpr int kMqaHG = 2;          // 16-head groups per workgroup
constexpr int kPlanWgs = 128;      // (query, split) pairs aimed at over the launch (two or more workgroups each)
constexpr int kPlanMinRows = 64;   // rows per split at least
constexpr int kMqaResidentWgs = 512;  // attention workgroups resident at once (two per CU)

void mqa_plan(int n_queries, int max_rows, int *n_splits, int *n_tiles) {
    // about kPlanWgs (query, split) pairs, at least kPlanMinRows rows (whole
    // tiles) per split; the tiles are dealt evenly, so splits differ by at most
    // one tile.  A single query takes one-tile splits: its launch stays small
    // (one 64K-token query's 640 rows: 20 splits, 40 workgroups; 27.4 against
    // 28.4 us for its fused step), while with four queries they measured slower.
    const int tiles = (max_rows + kTile - 1) / kTile;
    const int want_splits = (kPlanWgs + n_queries - 1) / n_queries;
    int s = tiles / ((n_queries == 1 ? kTile : kPlanMinRows) / kTile);
    if (s > want_splits) s = want_splits;
    if (s > kCombineMaxSplits) s = kCombineMaxSplits;
    if (s < 1) s = 1;
    *n_splits = s;
    *n_tiles = tiles > 0 ? tiles : 1;
}

size_t mqa_workspace_bytes(int dtype, int n_queries, int H, int D, int max_rows) {
    if (dtype != kBF16) return 0;
    int s, tiles;
    mqa_plan(n_queries, max_rows, &s, &tiles);
    if (s == 1) return 0;
    const size_t n = (size_t)n_queries * s * H;
    return n * D * 2 + n * 4 * 4 + 256;
}

void mqa_carve(MqaArgs &a, void *ws, int n_queries) {
    a.part_o = nullptr;
    a.part_ml = nullptr;
    if (a.n_splits <= 1) return;
    char *p = (char *)(((uintptr_t)ws + 255) & ~(uintptr_t)255);
    const size_t n = (size_t)n_queries * a.n_splits * a.H;
    a.part_o = p;
    a.part_ml = (float *)(p + n * a.D * 2);
}

hipError_t launch_mqa(const MqaArgs &a, int dtype, hipStream_t stream) {
    const int Q = a.B * a.T;
    if (dtype == kF32) {
        const size_t lds = sizeof(float) * (size_t)(a.D + 256);
        hipLaunchKernelGGL(mqa_f32_kernel, dim3(a.H, Q), dim3(256), lds, stream, a);
        return hipGetLastError();
    }
    const int Z = a.H / (16 * kMqaHG), pairs = a.n_splits * Q;
    const dim3 grid = (long)pairs * Z <= kMqaResidentWgs ? dim3(a.n_splits, Q, Z) : dim3((pairs + 7) / 8 * 8 * Z);
    const dim3 block(128 * kMqaHG);
    if (a.v != nullptr || a.win_v != nullptr)  // separate value rows
        hipLaunchKernelGGL((mqa_bf16_kernel<kMqaHG, true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((mqa_bf16_kernel<kMqaHG, false>), grid, block, 0, stream, a);
    if (a.n_splits > 1) {
        int zq = 1;  // dim parts of the combine: about 256 workgroups
        while (zq < 4 && (long)Q * (a.H / 4) * zq * 2 <= 256) zq *= 2;
        // many splits (the HCA layer): eight dim parts, so each thread folds fewer splits
        if (zq == 4 && a.n_splits >= 16 && (long)Q * (a.H / 4) * 8 <= 512) zq = 8;
        const dim3 grid(a.H / 4, Q, zq);
        if (zq == 8)
            hipLaunchKernelGGL(mqa_combine_kernel<8>, grid, dim3(256), 0, stream, a);
        else if (zq == 4)
            hipLaunchKernelGGL(mqa_combine_kernel<4>, grid, dim3(256), 0, stream, a);
        else if (zq == 2)
            hipLaunchKernelGGL(mqa_combine_kernel<2>, grid, dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL(mqa_combine_kernel<1>, grid, dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace csa
