// Accept kernel: one 64-lane wavefront per sequence, lane i <-> draft position i.
//
// Per lane: merge the vocabulary splits of draft row i and target row i into
// their log-normalisers, form the two log-probabilities of draft token t_i from
// the raw logits the row kernel recorded (FlashSpec technical summary,
// Methodology section 1: two log-probability scalars per candidate, one per
// model), draw the Philox block of (b, i) and
// run the log-space test log u < log p - log q in fp64. The first rejection is
// one ballot and a count of trailing zeros. The kernel writes the accepted
// prefix and the accept length, and leaves (k, u_res) for the residual kernel.
// Greedy sequences (T == 0) compare t_i with the target argmax instead and
// finish here. The verification outcome -- accepted count plus the extra
// token -- is what the Speculative Speculative Decoding summary (section 2,
// central concept, item 1) keys its speculation cache on.
//
// Also here: the scalar-only accept (O(B * gamma) bytes, nothing of size V)
// and the Philox test export.
#include <math.h>

#include "launch.hpp"
#include "philox.hpp"

namespace specv {
namespace {

__device__ inline double lse_of(const RowNorm& r) {
    return (static_cast<double>(r.m) + log2(r.s)) / static_cast<double>(kLog2e);
}

// The first kPre splits of a row are loaded up front with the kernel's other
// loads (one round trip to memory); further splits, if any, in the loop.
constexpr int kPre = 4;

struct RowSplits {
    Partial pre[kPre];
    const Partial* p;
    int nsplit;
    __device__ inline Partial at(int c) const { return c < kPre ? pre[c] : p[c]; }
};

__device__ inline void load_splits(RowSplits& r, const Partial* p, int nsplit) {
    r.p = p;
    r.nsplit = nsplit;
#pragma unroll
    for (int c = 0; c < kPre; ++c)
        r.pre[c] = p[c < nsplit ? c : nsplit - 1];  // unconditional, in range
}

__device__ inline bool merge_sampled(const RowSplits& r, RowNorm* out) {
    float m = kNegMax;
    for (int c = 0; c < r.nsplit; ++c)
        m = fmaxf(m, r.at(c).m);
    double s = 0.0;
    for (int c = 0; c < r.nsplit; ++c) {
        // exact 1 for the splits holding the max; a 1-ulp fp32 factor otherwise
        const Partial q = r.at(c);
        const float f = (q.m == m) ? 1.0f : fast_exp2(q.m - m);
        s = __builtin_fma(q.s, static_cast<double>(f), s);
    }
    *out = RowNorm{m, -1, s};
    return s > 0.0;  // false: the row has no finite logit
}

__device__ inline bool merge_greedy(const RowSplits& r, RowNorm* out) {
    float bv = -__builtin_huge_valf();
    int bi = 0x7fffffff;
    for (int c = 0; c < r.nsplit; ++c) {
        const Partial q = r.at(c);
        if (q.m > bv || (q.m == bv && q.idx < bi)) {
            bv = q.m;
            bi = q.idx;
        }
    }
    *out = RowNorm{bv, bi, 0.0};
    return bv > -__builtin_huge_valf();
}

template <int DT>
__global__ __launch_bounds__(64) void accept_kernel(
    const void* __restrict__ draft, const void* __restrict__ target,
    const int32_t* __restrict__ tokens, const float* __restrict__ temperature, int gamma,
    int vocab, int nsplit, uint64_t seed, uint64_t offset_arg,
    const uint64_t* __restrict__ offset_dev, const Partial* __restrict__ part,
    const float* __restrict__ gathered, RowNorm* __restrict__ rn, double* __restrict__ lse_out,
    SeqState* __restrict__ seq,
    int32_t* __restrict__ out_len, int32_t* __restrict__ out_tok) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int G = gamma;
    const int rps = 2 * G + 1;
    // The Philox offset: the argument, or a word in device memory that the
    // caller advances between replays of a captured call.
    const uint64_t offset = offset_dev ? offset_dev[0] : offset_arg;
    const size_t row0 = static_cast<size_t>(b) * rps;

    float inv_t = 0.0f;
    const int mode = temperature_mode(temperature[b], &inv_t);
    bool bad = mode < 0;
    const double nan = __builtin_nan("");

    // One pass over the positions, 64 at a time. Lane l handles position
    // i = i0 + l: it validates draft token t_i, merges the splits of draft row
    // i and target row i, gathers x_q[i][t_i] and x_p[i][t_i] (only for a valid
    // token) and decides acceptance. Lane l is the only lane that touches the
    // entries of rows i and G + i in rn and lse_out. Decisions made for a
    // sequence that turns out to be invalid are discarded below.
    int k = G;
    // coefficients of position k, broadcast from its lane once k is known
    float k_mp = 0.0f, k_mq = 0.0f, k_ratio = 1.0f;
    bool k_done = false;
    for (int i0 = 0; i0 <= G; i0 += 64) {
        const int i = i0 + lane;
        const bool has_draft = i < G;
        const bool has_target = i <= G;
        // Every load of this pass first, unconditional and clamped into range
        // (lanes past the sequence read position 0 or G and use nothing), so
        // they share one round trip instead of waiting on each other.
        const int id = has_draft ? i : 0;
        const int ip = has_target ? i : G;
        const int t_raw = G > 0 ? tokens[static_cast<size_t>(b) * G + id] : 0;
        const float zq_raw = gathered[row0 + id];
        const float zp_raw = gathered[row0 + G + ip];
        RowSplits sq, sp;
        load_splits(sq, part + (row0 + id) * nsplit, nsplit);
        load_splits(sp, part + (row0 + G + ip) * nsplit, nsplit);
        int t = 0;
        bool t_ok = false;
        if (has_draft) {
            t = t_raw;
            t_ok = t >= 0 && t < vocab;
            if (!t_ok)
                bad = true;
        }
        bool reject = false;
        RowNorm rq{0.0f, -1, 1.0}, rp{0.0f, -1, 1.0};
        if (mode == 1 && has_target) {
            // raw logits of the draft token, recorded by the row kernel
            const float zq = t_ok ? zq_raw : 0.0f;
            const float zp = t_ok ? zp_raw : 0.0f;
            if (has_draft) {
                if (!merge_sampled(sq, &rq))
                    bad = true;
                rn[row0 + i] = rq;
            }
            if (!merge_sampled(sp, &rp))
                bad = true;
            rn[row0 + G + i] = rp;
            const double lse_p = lse_of(rp);
            lse_out[row0 + G + i] = lse_p;
            if (has_draft) {
                const double lse_q = lse_of(rq);
                lse_out[row0 + i] = lse_q;
                const double lq = static_cast<double>(scale_logit(zq, inv_t)) - lse_q;
                const double lp = static_cast<double>(scale_logit(zp, inv_t)) - lse_p;
                const Words4 w = verify_block(seed, offset, static_cast<uint32_t>(b), static_cast<uint32_t>(i));
                const double log_u = log(static_cast<double>(uniform24(w.w0)));
                reject = !(log_u < lp - lq);
            }
        } else if (mode == 0 && has_target) {
            RowNorm rp;
            if (!merge_greedy(sp, &rp))
                bad = true;
            rn[row0 + G + i] = rp;
            if (has_draft) {
                lse_out[row0 + i] = nan;
                reject = t != rp.idx;
            }
            lse_out[row0 + G + i] = nan;
        } else if (has_target) {
            if (has_draft)
                lse_out[row0 + i] = nan;
            lse_out[row0 + G + i] = nan;
        }
        const unsigned long long mask = __ballot(reject);
        if (mask && k == G)
            k = i0 + __ffsll(static_cast<long long>(mask)) - 1;
        // position k lies in this pass: first rejection here, or no rejection
        // at all and this is the pass holding position G (wave-uniform test)
        if (!k_done && k >= i0 && k < i0 + 64 && (k < G || G < i0 + 64)) {
            const int src = k - i0;
            k_mp = __shfl(rp.m, src, 64);
            k_mq = __shfl(rq.m, src, 64);
            const double sp = __shfl(rp.s, src, 64), sq = __shfl(rq.s, src, 64);
            k_ratio = k < G ? static_cast<float>(sq / sp) : 1.0f;
            k_done = true;
        }
    }
    bad = __ballot(bad) != 0ull;

    if (bad) {
        for (int i = lane; i <= G; i += 64) {
            out_tok[static_cast<size_t>(b) * (G + 1) + i] = -1;
            if (i < G)
                lse_out[row0 + i] = nan;
            lse_out[row0 + G + i] = nan;
        }
        if (lane == 0) {
            out_len[b] = -1;
            // mode -1 marks a sentinel sequence for the kernels that follow
            seq[b] = SeqState{0, -1, 0.0f, 0.0f, 0.0f, 0.0f, 1.0f, 0};
        }
        return;
    }

    // Emit: accepted prefix, the greedy extra token, padding. The residual
    // kernels write the extra token of sampled sequences. Lane l reads back
    // only rows it wrote itself.
    for (int i = lane; i <= G; i += 64) {
        int v = -1;
        if (i < k)
            v = tokens[static_cast<size_t>(b) * G + i];
        else if (i == k && mode == 0)
            v = rn[row0 + G + k].idx;
        out_tok[static_cast<size_t>(b) * (G + 1) + i] = v;
    }
    if (lane == 0) {
        out_len[b] = k;
        const Words4 w = verify_block(seed, offset, static_cast<uint32_t>(b), static_cast<uint32_t>(k));
        seq[b] = SeqState{k, mode == 1 ? 1 : 0, uniform24(w.w1), inv_t, k_mp, k_mq, k_ratio, 0};
    }
}

__global__ __launch_bounds__(256) void accept_scalar_kernel(const float* __restrict__ logprobs,
                                                            int batch, int gamma, uint64_t seed,
                                                            uint64_t offset,
                                                            int32_t* __restrict__ out_len) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= batch)
        return;
    int k = gamma;
    for (int i = 0; i < gamma; ++i) {
        const float2 pr = reinterpret_cast<const float2*>(logprobs)[static_cast<size_t>(b) * gamma + i];
        const double d = static_cast<double>(pr.y) - static_cast<double>(pr.x);
        const Words4 w = verify_block(seed, offset, static_cast<uint32_t>(b), static_cast<uint32_t>(i));
        const double log_u = log(static_cast<double>(uniform24(w.w0)));
        if (!(log_u < d)) {
            k = i;
            break;
        }
    }
    out_len[b] = k;
}

__global__ __launch_bounds__(256) void philox_words_kernel(int batch, int gamma, uint64_t seed,
                                                           uint64_t offset, uint32_t* __restrict__ out) {
    const long n = static_cast<long>(batch) * (gamma + 1);
    const long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= n)
        return;
    const uint32_t b = static_cast<uint32_t>(t / (gamma + 1));
    const uint32_t i = static_cast<uint32_t>(t % (gamma + 1));
    const Words4 w = verify_block(seed, offset, b, i);
    reinterpret_cast<uint4*>(out)[t] = make_uint4(w.w0, w.w1, w.w2, w.w3);
}

}  // namespace

hipError_t launch_accept(const Shape& s, int nsplit, const void* draft, const void* target,
                         const int32_t* tokens, const float* temperature, uint64_t seed,
                         uint64_t offset, const uint64_t* offset_dev, const Partial* part,
                         const float* gathered, RowNorm* rn,
                         double* lse_out, SeqState* seq, int32_t* out_len, int32_t* out_tok,
                         hipStream_t stream, const LaunchEvents& ev) {
    if (s.batch == 0)
        return hipSuccess;
    return launch(s.dtype == kBF16 ? accept_kernel<kBF16> : accept_kernel<kF32>, dim3(s.batch),
                  dim3(64), 0, stream, ev, draft, target, tokens, temperature, s.gamma, s.vocab,
                  nsplit, seed, offset, offset_dev, part, gathered, rn, lse_out, seq, out_len,
                  out_tok);
}

hipError_t launch_accept_scalar(int batch, int gamma, const float* logprobs, uint64_t seed,
                                uint64_t offset, int32_t* out_len, hipStream_t stream) {
    if (batch == 0)
        return hipSuccess;
    const int blocks = (batch + 255) / 256;
    accept_scalar_kernel<<<dim3(blocks), dim3(256), 0, stream>>>(logprobs, batch, gamma, seed,
                                                                 offset, out_len);
    return hipGetLastError();
}

hipError_t launch_philox_words(int batch, int gamma, uint64_t seed, uint64_t offset,
                               uint32_t* out, hipStream_t stream) {
    const long n = static_cast<long>(batch) * (gamma + 1);
    if (n == 0)
        return hipSuccess;
    const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
    philox_words_kernel<<<dim3(blocks), dim3(256), 0, stream>>>(batch, gamma, seed, offset, out);
    return hipGetLastError();
}

}  // namespace specv
