// Constants and the activation shared by the indexer scorers (bf16 and fp8).
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace csa {

constexpr int kHI = 64;          // index heads of the MFMA scorers
constexpr int kDI = 128;         // index head dim of the MFMA scorers
constexpr int kScoreWaves = 4;   // waves per decode-scorer workgroup
constexpr int kTargetWgs = 256;  // decode scorers: about one workgroup per CU
constexpr int kEmitMax = 8192;   // entries of a stretch whose keys stay in LDS for the emission
constexpr int kEmitCapMax = 512; // emitted entries per workgroup at most
constexpr int kEmitTargetSlots = 4096;  // emitted slots per query the cap aims at, at least

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

// Entries per workgroup a decode scorer with the given step can hand the
// selection (its emitted entries), 0 if it cannot: every workgroup's stretch
// (at most ceil(steps / workgroups) steps) must fit in LDS, and the slots of
// all workgroups of a query must fit the selection and exceed K.
inline int decode_emit_cap(int n_max, int n_queries, int K, int wg_step) {
    const int wgs = decode_score_workgroups(n_max, n_queries, wg_step);
    const int steps = (n_max + wg_step - 1) / wg_step;
    const int chunk = (steps + wgs - 1) / wgs;
    if ((long)chunk * wg_step > kEmitMax) return 0;
    // about twice a workgroup's expected share of the K selected entries, plus a
    // margin, and at least an even share of 4,096 slots per query: with few
    // workgroups per query the threshold bin (1/8 octave) can hold more than K
    // entries, and a region that cannot emit all of its entries at or above it
    // sends the query to the slower whole-row selection (2 of the 32 queries of
    // a ragged batch at 64K-128K tokens did with 176 slots per region)
    int cap = (2 * K / wgs + 48 + 15) / 16 * 16;
    const int even = (kEmitTargetSlots / wgs + 15) / 16 * 16;
    cap = cap > even ? cap : even;
    cap = cap < 32 ? 32 : (cap > kEmitCapMax ? kEmitCapMax : cap);
    while (cap > 32 && (long)cap * wgs > kTopkMaxSlots) cap -= 16;
    // the selection's radix pass over the emitted slots needs more slots than K
    return (long)cap * wgs <= kTopkMaxSlots && (long)cap * wgs > K ? cap : 0;
}

}  // namespace csa
