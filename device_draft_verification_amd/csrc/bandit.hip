// Online draft-model selection on the device: one wavefront per bandit.
//
// A K-armed bandit chooses which draft model proposes the next tokens; the
// reward of a play is the fraction of draft tokens the verifier accepted, and
// the policy is UCB1 or Thompson sampling (FlashSpec technical summary,
// Methodology section 2). The kernel reads the verifier's accept lengths where
// they lie, folds them into the state of the arm each group played, and picks
// the next arm, all in one launch on the caller's stream.
//
// Layout of the work: one 64-lane wavefront per group. The lanes first stride
// over the group's accept lengths (integer sums, exact), then lane j owns arm
// j (K <= 64): its count and reward sum sit in registers for the update and
// the choice, and a butterfly over the wavefront finds the best arm.
//
// All arithmetic is IEEE double in source order (the library is built with
// contraction off), so the state after a step is the same bit pattern as any
// other implementation of the same formulas; a choice can only differ from
// another implementation's where two candidates, or a Marsaglia-Tsang test,
// are within the last few ulps of the transcendental functions.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <new>
#include <vector>

#include "philox.hpp"
#include "spec_bandit.h"

namespace specv {
namespace {

constexpr int kWave = 64;
constexpr int kMaxAttempts = 64;

struct BanditShape {
    int groups, arms, per_group, gamma, policy;
};

__device__ inline long long wave_sum_i64(long long v) {
#pragma unroll
    for (int m = 32; m > 0; m >>= 1)
        v += __shfl_xor(v, m, kWave);
    return v;
}

__device__ inline int wave_sum_i32(int v) {
#pragma unroll
    for (int m = 32; m > 0; m >>= 1)
        v += __shfl_xor(v, m, kWave);
    return v;
}

// Index of the largest score on the wavefront; the lowest index wins a tie.
__device__ inline int wave_argmax(double score, int idx) {
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) {
        const double os = __shfl_xor(score, m, kWave);
        const int oi = __shfl_xor(idx, m, kWave);
        if (os > score || (os == score && oi < idx)) {
            score = os;
            idx = oi;
        }
    }
    return idx;
}

// Gamma(shape, 1), shape >= 1, by Marsaglia and Tsang (ACM TOMS 26(3), 2000):
// d = shape - 1/3, c = 1/sqrt(9 d); a standard normal z (Box-Muller, cosine
// branch) and a uniform U are drawn until v = (1 + c z)^3 > 0 and
// ln U < z^2/2 + d - d v + d ln v; the variate is d v. The three uniforms of
// attempt a come from one Philox block whose first counter word carries the
// top bit, the arm, X or Y, and a; the second carries the group.
__device__ double gamma_variate(double shape, uint64_t seed, uint64_t offset, uint32_t group,
                                int arm, int which) {
    const double d = shape - 1.0 / 3.0;
    const double c = 1.0 / sqrt(9.0 * d);
    const double two_pi = 6.283185307179586;
    const double inv32 = 1.0 / 4294967296.0;
    const uint32_t base = 0x80000000u | static_cast<uint32_t>(kMaxAttempts * (2 * arm + which));
    for (int attempt = 0; attempt < kMaxAttempts; ++attempt) {
        const Words4 w = philox4x32_10(base + attempt, group, static_cast<uint32_t>(offset),
                                       static_cast<uint32_t>(offset >> 32),
                                       static_cast<uint32_t>(seed),
                                       static_cast<uint32_t>(seed >> 32));
        const double u1 = (static_cast<double>(w.w0) + 1.0) * inv32;
        const double u2 = static_cast<double>(w.w1) * inv32;
        const double uu = (static_cast<double>(w.w2) + 1.0) * inv32;
        const double z = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
        const double t = 1.0 + c * z;
        if (t <= 0.0)
            continue;
        const double v = t * t * t;
        const double lhs = log(uu);
        const double rhs = 0.5 * z * z + d - d * v + d * log(v);
        if (lhs < rhs)
            return d * v;
    }
    return d;
}

template <int POLICY>
__global__ __launch_bounds__(kWave) void bandit_step_kernel(
    BanditShape s, const int32_t* __restrict__ accept_len, const int32_t* arm_played,
    uint64_t seed, uint64_t offset, uint32_t* __restrict__ counts, double* __restrict__ sums,
    int32_t* out_arm) {
    const int g = blockIdx.x;
    const int lane = threadIdx.x;
    const long slot = static_cast<long>(g) * s.arms + lane;
    uint32_t n = 0;
    double sum = 0.0;
    if (lane < s.arms) {
        n = counts[slot];
        sum = sums[slot];
    }

    if (accept_len) {
        // arm_played may alias out_arm: every lane reads it before lane 0 writes.
        const int a = arm_played[g];
        if (a < 0 || a >= s.arms) {
            if (lane == 0)
                out_arm[g] = -1;
            return;
        }
        long long ksum = 0;
        int m = 0;
        const int b0 = g * s.per_group;
        for (int b = b0 + lane; b < b0 + s.per_group; b += kWave) {
            const int k = accept_len[b];
            if (k >= 0 && k <= s.gamma) {
                ksum += k;
                ++m;
            }
        }
        ksum = wave_sum_i64(ksum);
        m = wave_sum_i32(m);
        if (m > 0 && lane == a) {
            const double r = static_cast<double>(ksum) /
                             (static_cast<double>(s.gamma) * static_cast<double>(m));
            n += 1;
            sum += r;
            counts[slot] = n;
            sums[slot] = sum;
        }
    }

    int best;
    if (POLICY == SPEC_BANDIT_UCB1) {
        const unsigned long long unplayed = __ballot(lane < s.arms && n == 0);
        if (unplayed) {
            best = __ffsll(static_cast<long long>(unplayed)) - 1;
        } else {
            const long long total = wave_sum_i64(lane < s.arms ? static_cast<long long>(n) : 0);
            double score = -HUGE_VAL;
            if (lane < s.arms) {
                const double nj = static_cast<double>(n);
                const double mean = sum / nj;
                const double bonus = sqrt(2.0 * log(static_cast<double>(total)) / nj);
                score = mean + bonus;
            }
            best = wave_argmax(score, lane);
        }
    } else {
        double theta = -HUGE_VAL;
        if (lane < s.arms) {
            const double a = 1.0 + sum;
            const double b = 1.0 + (static_cast<double>(n) - sum);
            const double x = gamma_variate(a, seed, offset, g, lane, 0);
            const double y = gamma_variate(b, seed, offset, g, lane, 1);
            theta = x / (x + y);
        }
        best = wave_argmax(theta, lane);
    }
    if (lane == 0)
        out_arm[g] = best;
}

__global__ void bandit_fill_kernel(uint32_t* counts, double* sums, long n) {
    const long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) {
        counts[i] = 0;
        sums[i] = 0.0;
    }
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace
}  // namespace specv

using namespace specv;

struct spec_bandit_ctx {
    BanditShape shape{};
    hipStream_t stream = nullptr;
    void* state = nullptr;
    double* sums = nullptr;      // [G][K]
    uint32_t* counts = nullptr;  // [G][K]
};

extern "C" {

int spec_bandit_init(int n_groups, int n_arms, int batch, int gamma, int policy, void* hip_stream,
                     spec_bandit_ctx** out_ctx) {
    if (!out_ctx)
        return SPEC_EINVAL;
    *out_ctx = nullptr;
    if (n_groups < 1 || n_arms < 1 || n_arms > SPEC_BANDIT_MAX_ARMS || batch < 1 || gamma < 1 ||
        batch % n_groups != 0 ||
        (policy != SPEC_BANDIT_UCB1 && policy != SPEC_BANDIT_THOMPSON))
        return SPEC_EINVAL;
    spec_bandit_ctx* ctx = new (std::nothrow) spec_bandit_ctx();
    if (!ctx)
        return SPEC_ENOMEM;
    ctx->shape = BanditShape{n_groups, n_arms, batch / n_groups, gamma, policy};
    ctx->stream = static_cast<hipStream_t>(hip_stream);
    const size_t cells = static_cast<size_t>(n_groups) * n_arms;
    const size_t bytes = cells * (sizeof(double) + sizeof(uint32_t));
    if (hipMalloc(&ctx->state, bytes) != hipSuccess) {
        delete ctx;
        return SPEC_ENOMEM;
    }
    ctx->sums = static_cast<double*>(ctx->state);
    ctx->counts = reinterpret_cast<uint32_t*>(ctx->sums + cells);
    if (hipMemset(ctx->state, 0, bytes) != hipSuccess) {
        (void)hipFree(ctx->state);
        delete ctx;
        return SPEC_EHIP;
    }
    *out_ctx = ctx;
    return SPEC_OK;
}

int spec_bandit_set_stream(spec_bandit_ctx* ctx, void* hip_stream) {
    if (!ctx)
        return SPEC_EINVAL;
    ctx->stream = static_cast<hipStream_t>(hip_stream);
    return SPEC_OK;
}

int spec_bandit_step(spec_bandit_ctx* ctx, const int32_t* accept_len, const int32_t* arm_played,
                     uint64_t seed, uint64_t offset, int32_t* out_arm) {
    if (!ctx || !out_arm || !aligned4(out_arm))
        return SPEC_EINVAL;
    if (accept_len && (!arm_played || !aligned4(accept_len) || !aligned4(arm_played)))
        return SPEC_EINVAL;
    const BanditShape& s = ctx->shape;
    const dim3 grid(s.groups), block(kWave);
    if (s.policy == SPEC_BANDIT_UCB1)
        bandit_step_kernel<SPEC_BANDIT_UCB1><<<grid, block, 0, ctx->stream>>>(
            s, accept_len, accept_len ? arm_played : nullptr, seed, offset, ctx->counts, ctx->sums,
            out_arm);
    else
        bandit_step_kernel<SPEC_BANDIT_THOMPSON><<<grid, block, 0, ctx->stream>>>(
            s, accept_len, accept_len ? arm_played : nullptr, seed, offset, ctx->counts, ctx->sums,
            out_arm);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

int spec_bandit_get_state(spec_bandit_ctx* ctx, uint32_t* counts, double* sums) {
    if (!ctx || !counts || !sums)
        return SPEC_EINVAL;
    const size_t cells = static_cast<size_t>(ctx->shape.groups) * ctx->shape.arms;
    if (hipMemcpyAsync(counts, ctx->counts, cells * sizeof(uint32_t), hipMemcpyDeviceToHost,
                       ctx->stream) != hipSuccess ||
        hipMemcpyAsync(sums, ctx->sums, cells * sizeof(double), hipMemcpyDeviceToHost,
                       ctx->stream) != hipSuccess ||
        hipStreamSynchronize(ctx->stream) != hipSuccess)
        return SPEC_EHIP;
    return SPEC_OK;
}

int spec_bandit_set_state(spec_bandit_ctx* ctx, const uint32_t* counts, const double* sums) {
    if (!ctx || (!counts) != (!sums))
        return SPEC_EINVAL;
    const long cells = static_cast<long>(ctx->shape.groups) * ctx->shape.arms;
    if (!counts) {
        const int threads = 256;
        bandit_fill_kernel<<<dim3((cells + threads - 1) / threads), dim3(threads), 0,
                             ctx->stream>>>(ctx->counts, ctx->sums, cells);
        if (hipGetLastError() != hipSuccess || hipStreamSynchronize(ctx->stream) != hipSuccess)
            return SPEC_EHIP;
        return SPEC_OK;
    }
    for (long i = 0; i < cells; ++i)
        if (!(sums[i] >= 0.0 && sums[i] <= static_cast<double>(counts[i])))
            return SPEC_EINVAL;
    if (hipMemcpyAsync(ctx->counts, counts, cells * sizeof(uint32_t), hipMemcpyHostToDevice,
                       ctx->stream) != hipSuccess ||
        hipMemcpyAsync(ctx->sums, sums, cells * sizeof(double), hipMemcpyHostToDevice,
                       ctx->stream) != hipSuccess ||
        hipStreamSynchronize(ctx->stream) != hipSuccess)
        return SPEC_EHIP;
    return SPEC_OK;
}

int spec_bandit_destroy(spec_bandit_ctx* ctx) {
    if (!ctx)
        return SPEC_EINVAL;
    int rc = SPEC_OK;
    if (hipStreamSynchronize(ctx->stream) != hipSuccess)
        rc = SPEC_EHIP;
    if (ctx->state && hipFree(ctx->state) != hipSuccess)
        rc = SPEC_EHIP;
    delete ctx;
    return rc;
}

}  // extern "C"
