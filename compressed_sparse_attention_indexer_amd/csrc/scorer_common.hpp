// Constants and the activation shared by the indexer scorers (bf16 and fp8).
#pragma once

#include "common.hpp"
#include "launch.hpp"
#include "topk_hist.hpp"

namespace csa {

constexpr int kHI = 64;          // index heads of the MFMA scorers
constexpr int kDI = 128;         // index head dim of the MFMA scorers
constexpr int kScoreWaves = 4;   // waves per decode-scorer workgroup
constexpr int kTargetWgs = 256;  // decode scorers: about one workgroup per CU
constexpr int kEmitMax = 8192;   // entries of a stretch whose keys stay in LDS for the emission
constexpr int kEmitCapMax = 512; // emitted entries per workgroup at most
constexpr int kEmitTargetSlots = 4096;  // emitted slots per query the cap aims at, at least
constexpr int kBf16WgStep = kScoreWaves * 32;  // entries per workgroup step, bf16 decode scorer
constexpr int kFp8WgStep = kScoreWaves * 64;   // entries per workgroup step, fp8 decode scorer

// Indexer activation on an MFMA result: ReLU (kAct 0) or identity.  ReLU is
// a signed-integer max with 0 on the bit pattern (negative floats, -0.0
// included, are negative integers and become +0.0): one instruction, where
// fmaxf would first canonicalize its operand (MFMA results are not known to
// be canonical) and so take two.
template <int kAct>
__device__ __forceinline__ float index_act(float x) {
    return kAct == 0 ? __int_as_float(max(__float_as_int(x), 0)) : x;
}

// Decode-scorer workgroups per query: about one workgroup per CU over the
// launch, at most one per workgroup step of wg_step entries.
inline int decode_score_workgroups(int n_max, int n_queries, int wg_step) {
    int per_query = (kTargetWgs + n_queries - 1) / n_queries;
    const int steps = (n_max + wg_step - 1) / wg_step;
    if (per_query > steps) per_query = steps;
    return per_query < 1 ? 1 : per_query;
}

// End of a decode-scorer workgroup in the fused call, after its histogram
// window w is stored (that store's barrier also orders the LDS key writes):
// emit its region (the stretch's entries at or above a cut bin, at most em_cap
// of them, in index order), or mark the region overflowed if its stretch did
// not fit LDS (the host rules that out; the selection would then scan the row).
// `top` is the stretch's highest non-empty histogram bin (-1 if none), as the
// window store found it.
template <int NT>
__device__ void decode_emission(const ScoreArgs &a, const uint32_t *lh, const uint32_t *lkeys, bool emit, int nvis,
                                int s0, int n_load, int wg_step, size_t w, int top, int *s_scan, int *s_cut) {
    if (a.em_cap <= 0) return;
    const size_t r0 = w * a.em_cap;
    const int stretch0 = s0 * wg_step;
    if (emit) {
        int n_st = min(nvis, (s0 + n_load) * wg_step) - stretch0;
        n_st = n_st > 0 ? n_st : 0;
        emit_region<NT>(lh, lkeys, n_st, stretch0, a.em_cap, top, a.em_hdr + 2 * w, a.em_key + r0, a.em_idx + r0, s_scan,
                        s_cut);
    } else if (threadIdx.x == 0) {
        a.em_hdr[2 * w] = 0;
        a.em_hdr[2 * w + 1] = a.em_cap + 1;
    }
}

// Slots per region (workgroup) a decode scorer can hand the selection, for
// `wgs` region slots per query of up to `entries` entries each: about twice a
// workgroup's expected share of the K selected entries plus a margin for the
// members of the threshold bin (1/8 octave wide, so their number grows with
// the region: 48, or a sixteenth of a smaller region), and at least an even
// share of 4,096 slots per query (with few workgroups per query the threshold
// bin can hold more than K entries, and a region that cannot emit all of its
// entries at or above it sends the query to the slower whole-row selection: 2
// of the 32 queries of a ragged batch at 64K-128K tokens did with 176 slots per
// region).  On the synthetic decode inputs the most entries at or above the
// threshold bin in one region are 11 of 128 (one query at 64K tokens, 32
// slots), 33 of 4,096 (batch 4 at 1M, 64 slots), 52 of 4,096 (K = 1,024, 80
// slots) and 189 of 3,950 (ragged batch, 512 slots).  The slots of a query must
// fit the selection and exceed K.  0 if they cannot.
inline int decode_region_cap(int wgs, int K, long entries) {
    const int margin = entries / 16 < 48 ? (int)(entries / 16) : 48;
    int cap = (2 * K / wgs + margin + 15) / 16 * 16;
    const int even = (kEmitTargetSlots / wgs + 15) / 16 * 16;
    cap = cap > even ? cap : even;
    cap = cap < 32 ? 32 : (cap > kEmitCapMax ? kEmitCapMax : cap);
    while (cap > 32 && (long)cap * wgs > kTopkMaxSlots) cap -= 16;
    return (long)cap * wgs <= kTopkMaxSlots && (long)cap * wgs > K ? cap : 0;
}

// Geometry of a decode scorer in the fused call: P workgroups per query
// (about one per CU over the launch), one histogram window and one emitted
// region per workgroup; emission needs every workgroup's stretch (at most
// ceil(steps / P) steps) to fit kEmitMax entries.
inline DecodeGeom decode_geom_for(int n_max, int n_queries, int K, int step) {
    DecodeGeom g{};
    g.step = step;
    g.n_win = decode_score_workgroups(n_max, n_queries, step);
    const int steps = (n_max + step - 1) / step;
    const long stretch = (steps + g.n_win - 1) / g.n_win;
    g.em_cap = stretch * step <= kEmitMax ? decode_region_cap(g.n_win, K, stretch * step) : 0;
    return g;
}

}  // namespace csa
