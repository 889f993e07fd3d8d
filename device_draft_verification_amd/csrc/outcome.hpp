// Host-side launcher of the verification-outcome kernels (outcome.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace specv {

constexpr int kOutcomeMaxF = 64;       // longest list per length (one lane per entry)
constexpr int kOutcomeMaxSplit = 16;   // vocabulary splits per row pair

// One candidate of a top-F list: value and vocabulary index (-1: empty slot).
struct Cand {
    float v;
    int i;
};

// Work buffers of the outcome kernels, carved from the context's workspace:
// pairs * nsplit * F candidates and pairs * nsplit fp64 partial sums, with
// pairs = B * (G + 1).
struct OutcomeWork {
    Cand* cand;
    double* sums;
};

// Per (sequence, length) top-F of the extra token's distribution, its
// residual mass and the probability of the length, from the row normalisers,
// gathered logits and per-sequence state a verification call left behind.
// Two launches: B * (G + 1) * nsplit workgroups of kBlock threads, then one
// 64-lane wavefront per (sequence, length).
hipError_t launch_outcomes(const Shape& s, bool vec, int nsplit, int top_f, const void* draft,
                           const void* target, const int32_t* tokens, const SeqState* seq,
                           const RowNorm* rn, const double* lse, const float* gathered,
                           OutcomeWork work, int32_t* out_tok, float* out_prob, float* out_pk,
                           float* out_mass, hipStream_t stream);

}  // namespace specv
