// LSE merge arithmetic ("On Context Parallelism", section Peer-to-peer: merging completed
// attention tiles): merged = ln(e^a + e^c), weights e^(a - merged) and e^(c - merged).
// Shared by the merge kernel and the merging epilogue of the block kernels, so both give
// the same bits.  A side with lse = -inf weighs 0; two empty sides give (0, -inf).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

namespace cpattn {

struct MergeWeights {
    float w_old;  // weight of the accumulator
    float w_new;  // weight of the tile
    float lse;    // merged log-sum-exp
};

// Symmetric in (a, c): the larger operand anchors the log1p form.
__device__ inline MergeWeights merge_weights(float a, float c) {
    const float hi = fmaxf(a, c), lo = fminf(a, c);
    if (hi == -INFINITY) return MergeWeights{0.f, 0.f, -INFINITY};
    const float m = hi + log1pf(expf(lo - hi));
    return MergeWeights{expf(a - m), expf(c - m), m};
}

// w_old * x + w_new * y with two rounded products and a rounded sum (no fused multiply-add),
// so the result does not depend on which operand is the accumulator.
__device__ inline float merge_value(float x, float y, float w_old, float w_new) {
#pragma clang fp contract(off)
    return w_old * x + w_new * y;
}

}  // namespace cpattn
