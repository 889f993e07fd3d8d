// The accept step of one sequence, as a device function run by one 64-lane
// wavefront (lane i <-> draft position i): merge the vocabulary splits of
// draft row i and target row i into their log-normalisers, form the two
// log-probabilities of draft token t_i from the raw logits the row kernel
// recorded (FlashSpec technical summary, Methodology section 1: two
// log-probability scalars per candidate, one per model), draw the Philox
// block of (b, i) and run the log-space test log u < log p - log q in fp64.
// The first rejection is one ballot and a count of trailing zeros. Greedy
// sequences (T == 0) compare t_i with the target argmax instead. Used by the
// accept kernel, and folded into the draw's tile kernel for small batches.
#pragma once

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


// Decides sequence b; every lane returns its state (k, mode, the resample
// uniform and the coefficients of position k). With `write` it also stores
// the row normalisers, the log-normalisers, the accepted prefix (and the
// greedy extra token), the accept length and the state; without, nothing.
__device__ inline SeqState accept_sequence(const AcceptArgs& a, int b, bool write) {
    const int lane = threadIdx.x & 63;
    const int G = a.gamma;
    const int rps = 2 * G + 1;
    // The Philox offset: the argument, or a word in device memory that the
    // caller advances between replays of a captured call.
    const uint64_t offset = a.offset_dev ? a.offset_dev[0] : a.offset;
    const size_t row0 = static_cast<size_t>(b) * rps;

    float inv_t = 0.0f;
    const int mode = temperature_mode(a.temperature[b], &inv_t);
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
        const int t_raw = G > 0 ? a.tokens[static_cast<size_t>(b) * G + id] : 0;
        const float zq_raw = a.gathered[row0 + id];
        const float zp_raw = a.gathered[row0 + G + ip];
        RowSplits sq, sp;
        load_splits(sq, a.part + (row0 + id) * a.nsplit, a.nsplit);
        load_splits(sp, a.part + (row0 + G + ip) * a.nsplit, a.nsplit);
        int t = 0;
        bool t_ok = false;
        if (has_draft) {
            t = t_raw;
            t_ok = t >= 0 && t < a.vocab;
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
                if (write)
                    a.rn[row0 + i] = rq;
            }
            if (!merge_sampled(sp, &rp))
                bad = true;
            if (write)
                a.rn[row0 + G + i] = rp;
            const double lse_p = lse_of(rp);
            if (write)
                a.lse_out[row0 + G + i] = lse_p;
            if (has_draft) {
                const double lse_q = lse_of(rq);
                if (write)
                    a.lse_out[row0 + i] = lse_q;
                const double lq = static_cast<double>(scale_logit(zq, inv_t)) - lse_q;
                const double lp = static_cast<double>(scale_logit(zp, inv_t)) - lse_p;
                const Words4 w = verify_block(a.seed, offset, static_cast<uint32_t>(b), static_cast<uint32_t>(i));
                const double log_u = log(static_cast<double>(uniform24(w.w0)));
                reject = !(log_u < lp - lq);
            }
        } else if (mode == 0 && has_target) {
            RowNorm rp;
            if (!merge_greedy(sp, &rp))
                bad = true;
            if (write) {
                a.rn[row0 + G + i] = rp;
                if (has_draft)
                    a.lse_out[row0 + i] = nan;
                a.lse_out[row0 + G + i] = nan;
            }
            if (has_draft)
                reject = t != rp.idx;
        } else if (has_target && write) {
            if (has_draft)
                a.lse_out[row0 + i] = nan;
            a.lse_out[row0 + G + i] = nan;
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
        // mode -1 marks a sentinel sequence for the kernels that follow
        const SeqState st{0, -1, 0.0f, 0.0f, 0.0f, 0.0f, 1.0f, 0};
        if (write) {
            for (int i = lane; i <= G; i += 64) {
                a.out_tok[static_cast<size_t>(b) * (G + 1) + i] = -1;
                if (i < G)
                    a.lse_out[row0 + i] = nan;
                a.lse_out[row0 + G + i] = nan;
            }
            if (lane == 0) {
                a.out_len[b] = -1;
                a.seq[b] = st;
            }
        }
        return st;
    }

    // Emit: accepted prefix, the greedy extra token, padding. The residual
    // kernels write the extra token of sampled sequences. Lane l reads back
    // only rows it wrote itself.
    const Words4 w = verify_block(a.seed, offset, static_cast<uint32_t>(b), static_cast<uint32_t>(k));
    const SeqState st{k, mode == 1 ? 1 : 0, uniform24(w.w1), inv_t, k_mp, k_mq, k_ratio, 0};
    if (write) {
        for (int i = lane; i <= G; i += 64) {
            int v = -1;
            if (i < k)
                v = a.tokens[static_cast<size_t>(b) * G + i];
            else if (i == k && mode == 0)
                v = a.rn[row0 + G + k].idx;
            a.out_tok[static_cast<size_t>(b) * (G + 1) + i] = v;
        }
        if (lane == 0) {
            a.out_len[b] = k;
            a.seq[b] = st;
        }
    }
    return st;
}

}  // namespace
}  // namespace specv
