// Constants and the activation shared by the indexer scorers (bf16 and fp8).
#pragma once

#include "common.hpp"

namespace csa {

constexpr int kHI = 64;          // index heads of the MFMA scorers
constexpr int kDI = 128;         // index head dim of the MFMA scorers
constexpr int kScoreWaves = 4;   // waves per decode-scorer workgroup
constexpr int kTargetWgs = 256;  // decode scorers: about one workgroup per CU

// Indexer activation on an MFMA result: ReLU (kAct 0) or identity.  ReLU is
// a signed-integer max with 0 on the bit pattern (negative floats, -0.0
// included, are negative integers and become +0.0): one instruction, where
// fmaxf would first canonicalize its operand (MFMA results are not known to
// be canonical) and so take two.
template <int kAct>
__device__ __forceinline__ float index_act(float x) {
    return kAct == 0 ? __int_as_float(max(__float_as_int(x), 0)) : x;
}

}  // namespace csa
