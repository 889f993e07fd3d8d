// Verification-outcome kernels: for every sequence and every possible accept
// length i in [0, G], the F most likely extra tokens with their probabilities,
// the residual mass S_i, and the probability of that length given the drafts.
//
// The outcome of a verification -- accepted count plus extra token -- is what
// speculative speculative decoding predicts and keys its speculation cache on;
// Saguaro spends the cache on likely lengths and, per length, on the top-F
// tokens of the residual distribution the extra token is drawn from
// (Speculative Speculative Decoding summary, section 2: central concept, and
// Saguaro challenges 1 and 2). With the drafts fixed the law is exact:
//   beta_j = min(1, p_j(t_j) / q_j(t_j)),
//   P(k = i) = prod_{j<i} beta_j * (1 - beta_i), P(k = G) = prod_j beta_j,
//   extra | k = i ~ max(0, p_i - q_i) / S_i (i < G), p_G (i = G), p_i if S_i = 0;
// greedy sequences have a deterministic outcome (lists by raw target logit).
//
// Work layout.
//   outcome_topf: grid = B * (G+1) * nsplit workgroups of four wavefronts; a
//     workgroup streams one vocabulary split of target row i and draft row i
//     (lane l reads group 64 t + l of a tile t, so a load instruction covers
//     1 KiB of consecutive memory) and evaluates the scaled residual
//     r' = max(0, p' * s_q / s_p - q') with p' = 2^(x log2e - m_p), the same
//     arithmetic as the residual draw. Each wavefront keeps a candidate list
//     in LDS behind a threshold that only rises: a group whose largest value
//     reaches it appends its values that beat the threshold key (one prefix
//     count over the lanes places every lane's run, no atomics). The threshold is seeded from the
//     first batch (the F-th largest of the lanes' maxima is a lower bound of
//     the F-th largest element), raised to the F-th best key whenever the
//     list is cut back to F (once it holds more than kTightenAt), and shared
//     by the workgroup's four wavefronts: each one's threshold bounds the
//     workgroup's F-th best from below, so all filter by the largest.
//     The four wavefront lists are merged by wavefront 0 into F candidates
//     and one fp64 partial sum per split.
//   outcome_merge: one wavefront per (sequence, length) merges the splits,
//     normalises, and forms P(k = i) from the accept test's log-probabilities.
// Keys order by value, then by lower vocabulary index, so the lists are those
// of a stable descending sort.
#include <math.h>

#include "outcome.hpp"
#include "spec_verify.h"

namespace specv {
namespace {

constexpr int kTightenAt = 32;  // the list is cut back to F once it holds more
// Candidate slots per wavefront: a list is at most max(kTightenAt, F) long
// before a tile (a cut keeps F), and one tile adds at most 64 * 8 values.
constexpr int kCap = (kTightenAt > kOutcomeMaxF ? kTightenAt : kOutcomeMaxF) + 64 * 8;
// the merge kernel's list: every split's F candidates
constexpr int kMergeCap = kOutcomeMaxSplit * kOutcomeMaxF;
constexpr int kIdxNone = 0x7fffffff;

__device__ __forceinline__ bool key_gt(float v, int i, float tv, int ti) {
    return v > tv || (v == tv && i < ti);
}

__device__ inline int lane_id() { return threadIdx.x & 63; }

// Bitonic sort of one key per lane across the wavefront, largest key first.
__device__ __forceinline__ void wave_sort_desc(float& v, int& i) {
    const int lane = lane_id();
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const float ov = __shfl_xor(v, j, 64);
            const int oi = __shfl_xor(i, j, 64);
            const bool keep_max = ((lane & j) == 0) == ((lane & k) == 0);
            const bool take = keep_max ? key_gt(ov, oi, v, i) : key_gt(v, i, ov, oi);
            if (take) {
                v = ov;
                i = oi;
            }
        }
    }
}

__device__ inline double wave_sum_f64(double v) {
#pragma unroll
    for (int m = 32; m > 0; m >>= 1)
        v += __shfl_xor(v, m, 64);
    return v;
}

__device__ inline double wave_prod_f64(double v) {
#pragma unroll
    for (int m = 32; m > 0; m >>= 1)
        v *= __shfl_xor(v, m, 64);
    return v;
}

// A wavefront's candidate list in LDS and its threshold key (wave-uniform).
struct WaveList {
    Cand* buf;
    int count;
    float tv;
    int ti;
    // The workgroup's thresholds, one key per wavefront (NULL: not shared).
    // Every wavefront's threshold is at most the F-th best key it has seen,
    // so the largest of them bounds the F-th best of the whole workgroup from
    // below, and a wavefront may filter by it.
    unsigned long long* shared;
    int wid;
};

// Inclusive prefix of an int over the wavefront's lanes (lane order) by DPP
// moves: shifts by 1, 2, 4, 8 within each row of 16 lanes, then the row
// broadcasts carry the row totals forward.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int add_dpp_i(int v) {
    return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, true);
}

__device__ __forceinline__ int wave_inclusive_scan_i(int v) {
    v = add_dpp_i<0x111, 0xF>(v);  // row_shr:1
    v = add_dpp_i<0x112, 0xF>(v);  // row_shr:2
    v = add_dpp_i<0x114, 0xF>(v);  // row_shr:4
    v = add_dpp_i<0x118, 0xF>(v);  // row_shr:8
    v = add_dpp_i<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v = add_dpp_i<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

// Append every value of the lane's group that reaches the threshold value
// (a superset of the entries at or above the threshold key, which the cuts
// sort out), lane after lane: one prefix count over the lanes places each
// lane's run, so the whole group costs one scan instead of one ballot per
// element.
template <int W>
__device__ __forceinline__ void append_group(WaveList& L, bool used, const float (&val)[W], int idx0) {
    // An element tied with the threshold value beats the threshold key only
    // below its index: a group whose indices all lie at or past it compares
    // with the next float up instead. Without this, a value shared by many
    // elements (an exact 0 of the residual, a common bf16 logit) lets every
    // one of them in and the list is cut on every group.
    float tq = L.tv;
    if (L.ti <= idx0) {
        const uint32_t u = __float_as_uint(L.tv);
        tq = (u << 1) == 0 ? __uint_as_float(1u) : __uint_as_float((u >> 31) ? u - 1 : u + 1);
    }
    int c = 0;
#pragma unroll
    for (int e = 0; e < W; ++e)
        c += (used && val[e] >= tq) ? 1 : 0;
    const int incl = wave_inclusive_scan_i(c);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    int pos = L.count + incl - c;
#pragma unroll
    for (int e = 0; e < W; ++e) {
        if (used && val[e] >= tq) {
            L.buf[pos] = Cand{val[e], idx0 + e};
            ++pos;
        }
    }
    L.count += total;
}

// Keys as 64-bit unsigned integers that order like (value, then lower index):
// the value's bits mapped to an order-preserving code in the high word, the
// complemented index in the low word. -0 is coded as +0, so the codes agree
// with floating-point equality. 0 is below every real key.
__device__ __forceinline__ uint64_t key_code(float v, int idx) {
    uint32_t u = __float_as_uint(v);
    if ((u << 1) == 0)
        u = 0;
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (static_cast<uint64_t>(o) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(idx));
}

__device__ __forceinline__ void key_decode(uint64_t k, float* v, int* idx) {
    const uint32_t o = static_cast<uint32_t>(k >> 32);
    const uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
    *v = __uint_as_float(u);
    *idx = static_cast<int>(~static_cast<uint32_t>(k));
}

// Publish this wavefront's threshold to its workgroup.
__device__ __forceinline__ void publish_threshold(const WaveList& L) {
    if (L.shared && lane_id() == 0)
        __hip_atomic_store(L.shared + L.wid, key_code(L.tv, L.ti), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Take the workgroup's largest threshold when it is above this wavefront's
// (slots start at 0, below every key).
__device__ __forceinline__ void adopt_threshold(WaveList& L) {
    if (!L.shared)
        return;
    unsigned long long k = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const unsigned long long o =
            __hip_atomic_load(L.shared + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        k = o > k ? o : k;
    }
    if (k > key_code(L.tv, L.ti))
        key_decode(k, &L.tv, &L.ti);
}

// Cut the list to its F best candidates (unordered) and raise the threshold
// to the F-th best key. The F-th best is found by binary searches over the key
// bits with ballot counts, so no data moves between lanes: first over the
// value code (the largest h with at least F keys of value code >= h), then,
// only if several candidates share that value and not all of them fit, over
// the index among those. Fewer than F candidates: all are kept.
// Slots are read S per lane from registers when the list fits 64 * S slots,
// else from LDS on every step (a rare path: lists are cut once they pass 64).
template <int S>
struct SlotKeys {
    uint32_t hi[S], lo[S];
};

template <int S>
__device__ __forceinline__ void load_keys(const WaveList& L, SlotKeys<S>& K) {
    const int lane = lane_id();
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int slot = s * 64 + lane;
        K.hi[s] = 0;
        K.lo[s] = 0;
        if (slot < L.count) {
            const Cand c = L.buf[slot];
            if (c.i >= 0) {
                const uint64_t k = key_code(c.v, c.i);
                K.hi[s] = static_cast<uint32_t>(k >> 32);
                K.lo[s] = static_cast<uint32_t>(k);
            }
        }
    }
}

// count of slots with (hi > h) or (hi == h and lo >= l); `eq_only` counts only hi == h
template <int S>
__device__ __forceinline__ int count_ge(const SlotKeys<S>& K, uint32_t h, uint32_t l, bool eq_only) {
    int n = 0;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const bool ge = eq_only ? (K.hi[s] == h && K.lo[s] >= l)
                                : (K.hi[s] > h || (K.hi[s] == h && K.lo[s] >= l));
        n += __popcll(__ballot(ge));
    }
    return n;
}

__device__ __forceinline__ int count_ge_lds(const WaveList& L, uint32_t h, uint32_t l, bool eq_only) {
    const int lane = lane_id();
    int n = 0;
    for (int base = 0; base < L.count; base += 64) {
        const int slot = base + lane;
        bool ge = false;
        if (slot < L.count) {
            const Cand c = L.buf[slot];
            if (c.i >= 0) {
                const uint64_t k = key_code(c.v, c.i);
                const uint32_t kh = static_cast<uint32_t>(k >> 32), kl = static_cast<uint32_t>(k);
                ge = eq_only ? (kh == h && kl >= l) : (kh > h || (kh == h && kl >= l));
            }
        }
        n += __popcll(__ballot(ge));
    }
    return n;
}

template <int S, typename KT>
__device__ __forceinline__ int count_keys(const WaveList& L, const KT& K, uint32_t h,
                                          uint32_t l, bool eq_only) {
    if constexpr (S > 0)
        return count_ge(K, h, l, eq_only);
    else
        return count_ge_lds(L, h, l, eq_only);
}

template <int S>
__device__ __forceinline__ void tighten_s(WaveList& L, int F) {
    SlotKeys<(S > 0 ? S : 1)> K;
    if constexpr (S > 0)
        load_keys(L, K);
    // value code of the F-th best
    uint32_t h = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t c = h | (1u << bit);
        if (count_keys<S>(L, K, c, 0u, false) >= F)
            h = c;
    }
    uint32_t l = 0;      // keep (hi, lo) >= (h, l)
    bool exact = false;  // the threshold index is the F-th's own
    if (h != 0) {
        const int n_ge = count_keys<S>(L, K, h, 0u, false);
        if (n_ge > F) {
            // more candidates share value h than fit: search their index word
            const int n_gt = n_ge - count_keys<S>(L, K, h, 0u, true);
            const int need = F - n_gt;
            for (int bit = 31; bit >= 0; --bit) {
                const uint32_t c = l | (1u << bit);
                if (count_keys<S>(L, K, h, c, true) >= need)
                    l = c;
            }
            exact = true;
        }
    } else {
        h = 0;
        l = 1;  // fewer than F candidates: keep every real key
    }
    // Compact the kept slots to the front, in slot order. A slot is written at
    // or below its own position, and every lane reads its slot of a row before
    // any lane writes in that row, so nothing unread is overwritten.
    const int lane = lane_id();
    int n = 0;
    const int count = L.count;
    for (int base = 0; base < count; base += 64) {
        const int slot = base + lane;
        Cand c{0.0f, -1};
        bool keep = false;
        if (slot < count) {
            c = L.buf[slot];
            if (c.i >= 0) {
                const uint64_t k = key_code(c.v, c.i);
                const uint32_t kh = static_cast<uint32_t>(k >> 32), kl = static_cast<uint32_t>(k);
                keep = kh > h || (kh == h && kl >= l);
            }
        }
        const unsigned long long m = __ballot(keep);
        __builtin_amdgcn_wave_barrier();
        if (keep) {
            const int below = __builtin_amdgcn_mbcnt_hi(static_cast<unsigned>(m >> 32),
                                                        __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(m), 0));
            L.buf[n + below] = c;
        }
        n += __popcll(m);
    }
    __builtin_amdgcn_wave_barrier();
    L.count = n;
    if (h != 0 && n >= F) {
        // threshold: the F-th key itself, or the lowest key of its value
        key_decode((static_cast<uint64_t>(h) << 32) | (exact ? l : 0u), &L.tv, &L.ti);
        if (!exact)
            L.ti = kIdxNone;
    }
}

template <int SMAX>
__device__ __forceinline__ void tighten(WaveList& L, int F) {
    if (L.count <= F)
        return;
    if (L.count <= 64)
        tighten_s<1>(L, F);
    else if (L.count <= 256)
        tighten_s<4>(L, F);
    else
        tighten_s<0>(L, F);
}

// The list (at most 64 entries after tighten) sorted by key, largest first,
// one entry per lane: lane j holds entry j, or (-inf, -1) past the end.
__device__ __forceinline__ void sorted_entries(const WaveList& L, float* v, int* i) {
    const int lane = lane_id();
    float vv = -__builtin_huge_valf();
    int ii = kIdxNone;
    if (lane < L.count) {
        const Cand c = L.buf[lane];
        if (c.i >= 0) {
            vv = c.v;
            ii = c.i;
        }
    }
    wave_sort_desc(vv, ii);
    if (ii == kIdxNone)
        ii = -1;
    *v = vv;
    *i = ii;
}

// What ranks the entries of a row pair: the raw target logit (greedy
// sequences), p' alone (bonus row, or the empty-residual fallback), or the
// scaled residual.
enum Kind { kRaw = 0, kP = 1, kResidual = 2 };

struct RowCoefs {
    const void* prow;
    const void* qrow;
    int kind;
    float inv_t, mp, mq, ratio;
};

template <int DT, bool VEC, int KIND>
__device__ inline void group_values(const RowCoefs& rc, const typename Loader<DT, VEC>::raw_t& p,
                                    const typename Loader<DT, VEC>::raw_t& q,
                                    float (&val)[Loader<DT, VEC>::W]) {
    using Ld = Loader<DT, VEC>;
    constexpr int W = Ld::W;
    float zp[W];
    Ld::unpack(p, zp);
    if constexpr (KIND == kRaw) {
#pragma unroll
        for (int e = 0; e < W; ++e)
            val[e] = zp[e];
    } else if constexpr (KIND == kP) {
#pragma unroll
        for (int e = 0; e < W; ++e)
            val[e] = fast_exp2(__builtin_fmaf(scale_logit(zp[e], rc.inv_t), kLog2e, -rc.mp));
    } else {
        float zq[W];
        Ld::unpack(q, zq);
#pragma unroll
        for (int e = 0; e < W; ++e) {
            const float pv = fast_exp2(__builtin_fmaf(scale_logit(zp[e], rc.inv_t), kLog2e, -rc.mp));
            const float qv = fast_exp2(__builtin_fmaf(scale_logit(zq[e], rc.inv_t), kLog2e, -rc.mq));
            val[e] = fmaxf(__builtin_fmaf(pv, rc.ratio, -qv), 0.0f);
        }
    }
}

template <int N>
__device__ inline float pairwise_sum(const float (&r)[N]) {
    float t[N];
#pragma unroll
    for (int e = 0; e < N; ++e)
        t[e] = r[e];
#pragma unroll
    for (int w = 1; w < N; w <<= 1) {
#pragma unroll
        for (int i = 0; i + w < N; i += 2 * w)
            t[i] += t[i + w];
    }
    return t[0];
}

template <int N>
__device__ inline float group_max(const float (&r)[N]) {
    float m = r[0];
#pragma unroll
    for (int e = 1; e < N; ++e)
        m = fmaxf(m, r[e]);
    return m;
}

// One wavefront streams tiles t_begin, t_begin + t_step, ... (< t_end) of a
// row pair into its list and returns its fp64 sum of the values (KIND > kRaw).
// Double-buffered: the U tiles of the next batch are loaded, unconditionally
// (past the end they read group 0, which is in cache, and are never used),
// before the current batch is consumed, so the compiler waits for exactly the
// group being consumed. A group enters the list only if its largest value
// reaches the threshold, which is one compare per group in the common case.
template <int DT, bool VEC, bool NT, int KIND, int U>
__device__ __forceinline__ double stream_tiles(const RowCoefs& rc, int groups, int t_begin, int t_end, int t_step,
                               int F, WaveList& L) {
    using Ld = Loader<DT, VEC>;
    using raw_t = typename Ld::raw_t;
    constexpr int W = Ld::W;
    const int lane = lane_id();
    double sum = 0.0;
    bool seeded = false;
    auto load_batch = [&](raw_t (&p)[U], raw_t (&q)[U], int t) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tt = t + u * t_step;
            const int g = tt * 64 + lane;
            const bool used = tt < t_end && g < groups;
            p[u] = Ld::template load_as<NT>(rc.prow, used ? g : 0);
            if constexpr (KIND == kResidual)
                q[u] = Ld::template load_as<NT>(rc.qrow, used ? g : 0);
        }
    };
    auto consume = [&](const raw_t (&p)[U], const raw_t (&q)[U], int t) {
        float val[U][W];
        bool used[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            group_values<DT, VEC, KIND>(rc, p[u], q[u], val[u]);
            const int tt = t + u * t_step;
            used[u] = tt < t_end && tt * 64 + lane < groups;
        }
        if constexpr (KIND != kRaw) {
            float bs = 0.0f;  // one batch of one lane: at most 32 values
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (used[u])
                    bs += pairwise_sum(val[u]);
            sum += static_cast<double>(bs);
        }
        if (!seeded) {
            // Threshold seed from the first batch: the F-th largest of the
            // lanes' best values is a lower bound of the F-th largest element.
            uint32_t best = 0;
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (used[u]) {
                    const uint32_t c = static_cast<uint32_t>(key_code(group_max(val[u]), 0) >> 32);
                    best = c > best ? c : best;
                }
            uint32_t h = 0;
            for (int bit = 31; bit >= 0; --bit) {
                const uint32_t c = h | (1u << bit);
                if (__popcll(__ballot(best >= c)) >= F)
                    h = c;
            }
            if (h != 0) {
                key_decode(static_cast<uint64_t>(h) << 32, &L.tv, &L.ti);
                L.ti = kIdxNone;  // the lowest key of that value
            }
            seeded = true;
            publish_threshold(L);
        }
        adopt_threshold(L);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (__ballot(used[u] && group_max(val[u]) >= L.tv)) {
                const int g = (t + u * t_step) * 64 + lane;
                append_group<W>(L, used[u], val[u], g * W);
                if (L.count > kTightenAt) {
                    tighten<kCap / 64>(L, F);
                    publish_threshold(L);
                }
            }
        }
    };
    raw_t pa[U], qa[U], pb[U], qb[U];
    const int step = U * t_step;
    int t = t_begin;
    if (t >= t_end)
        return sum;
    // Batches in pairs with no exit between the halves: at the loop head only
    // the a-batch's loads are in flight, so the compiler waits for exactly the
    // batch being consumed (a mid-loop exit makes it wait for everything).
    const int nb = (t_end - t + step - 1) / step;
    load_batch(pa, qa, t);
    for (int i = 0; i + 2 <= nb; i += 2) {
        load_batch(pb, qb, t + step);
        consume(pa, qa, t);
        load_batch(pa, qa, t + 2 * step);
        consume(pb, qb, t + step);
        t += 2 * step;
    }
    if (nb & 1)
        consume(pa, qa, t);
    return sum;
}

template <int DT, bool VEC, bool NT, int U>
__device__ __forceinline__ double stream_pair(const RowCoefs& rc, int groups, int t_begin, int t_end,
                                     int t_step, int F, WaveList& L) {
    if (rc.kind == kResidual)
        return stream_tiles<DT, VEC, NT, kResidual, U>(rc, groups, t_begin, t_end, t_step, F, L);
    if (rc.kind == kP)
        return stream_tiles<DT, VEC, NT, kP, U>(rc, groups, t_begin, t_end, t_step, F, L);
    return stream_tiles<DT, VEC, NT, kRaw, U>(rc, groups, t_begin, t_end, t_step, F, L);
}

// Coefficients of row pair (b, i): target row i and, for a residual, draft row i.
template <int DT>
__device__ inline RowCoefs pair_coefs(const void* draft, const void* target, int G, int vocab,
                                      int b, int i, const SeqState& st, const RowNorm* rn) {
    RowCoefs rc;
    const size_t row0 = static_cast<size_t>(b) * (2 * G + 1);
    rc.prow = row_ptr(target, DT, static_cast<size_t>(b) * (G + 1) + i, vocab);
    rc.qrow = rc.prow;
    rc.inv_t = st.inv_t;
    rc.mp = rc.mq = 0.0f;
    rc.ratio = 1.0f;
    if (st.mode == 0) {
        rc.kind = kRaw;
        return rc;
    }
    const RowNorm rp = rn[row0 + G + i];
    rc.mp = rp.m;
    if (i == G) {
        rc.kind = kP;
        return rc;
    }
    const RowNorm rq = rn[row0 + i];
    rc.kind = kResidual;
    rc.qrow = row_ptr(draft, DT, static_cast<size_t>(b) * G + i, vocab);
    rc.mq = rq.m;
    rc.ratio = static_cast<float>(rq.s / rp.s);
    return rc;
}

template <int DT, bool VEC, bool NT>
__global__ __launch_bounds__(kBlock) void outcome_topf_kernel(
    const void* __restrict__ draft, const void* __restrict__ target, int gamma, int vocab,
    int nsplit, int tiles_per_split, int F, const SeqState* __restrict__ seq,
    const RowNorm* __restrict__ rn, Cand* __restrict__ cand_out, double* __restrict__ sum_out) {
    constexpr int W = Loader<DT, VEC>::W;
    __shared__ Cand lds[kWaves][kCap];
    __shared__ double lds_sum[kWaves];
    __shared__ int lds_n[kWaves];
    __shared__ unsigned long long lds_thr[kWaves];
    const int pair = blockIdx.x / nsplit;
    const int c = blockIdx.x - pair * nsplit;
    const int G = gamma;
    const int b = pair / (G + 1);
    const int i = pair - b * (G + 1);
    const SeqState st = seq[b];
    if (st.mode < 0)
        return;  // sentinel sequence: the merge kernel writes its outputs
    const RowCoefs rc = pair_coefs<DT>(draft, target, G, vocab, b, i, st, rn);
    const int groups = vocab / W;
    const int ntiles = (groups + 63) / 64;
    const int t0 = c * tiles_per_split;
    const int t1 = t0 + tiles_per_split < ntiles ? t0 + tiles_per_split : ntiles;
    const int wid = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int lane = lane_id();

    if (threadIdx.x < kWaves)
        lds_thr[threadIdx.x] = 0;
    __syncthreads();
    WaveList L{lds[wid], 0, -__builtin_huge_valf(), kIdxNone, lds_thr, wid};
    double sum = stream_pair<DT, VEC, NT, 4>(rc, groups, t0 + wid, t1, kWaves, F, L);
    tighten<kCap / 64>(L, F);
    sum = wave_sum_f64(sum);
    if (lane == 0) {
        lds_sum[wid] = sum;
        lds_n[wid] = L.count;
    }
    __syncthreads();
    if (wid != 0)
        return;
    int total = lds_n[0];
    for (int w = 1; w < kWaves; ++w) {
        const int n = lds_n[w];
        if (lane < n)
            L.buf[total + lane] = lds[w][lane];
        total += n;
    }
    __builtin_amdgcn_wave_barrier();
    L.count = total;
    tighten<kCap / 64>(L, F);
    const int n = L.count;
    Cand* out = cand_out + (static_cast<size_t>(pair) * nsplit + c) * F;
    if (lane < F)
        out[lane] = lane < n ? L.buf[lane] : Cand{-__builtin_huge_valf(), -1};
    if (lane == 0)
        sum_out[static_cast<size_t>(pair) * nsplit + c] =
            ((lds_sum[0] + lds_sum[1]) + lds_sum[2]) + lds_sum[3];
}

// beta_j = min(1, p_j(t_j) / q_j(t_j)) from the accept test's log-probabilities
// (0 when the difference is NaN); for greedy sequences 1 iff t_j is the argmax.
__device__ inline double accept_prob(int j, int b, int G, int mode, float inv_t,
                                     const int32_t* tokens, const RowNorm* rn, const double* lse,
                                     const float* gathered) {
    const size_t row0 = static_cast<size_t>(b) * (2 * G + 1);
    if (mode == 0)
        return tokens[static_cast<size_t>(b) * G + j] == rn[row0 + G + j].idx ? 1.0 : 0.0;
    const double lq = static_cast<double>(scale_logit(gathered[row0 + j], inv_t)) - lse[row0 + j];
    const double lp = static_cast<double>(scale_logit(gathered[row0 + G + j], inv_t)) - lse[row0 + G + j];
    const double d = lp - lq;
    return d >= 0.0 ? 1.0 : (d < 0.0 ? exp(d) : 0.0);
}

template <int DT, bool VEC>
__global__ __launch_bounds__(64) void outcome_merge_kernel(
    const void* __restrict__ draft, const void* __restrict__ target,
    const int32_t* __restrict__ tokens, int gamma, int vocab, int nsplit, int F,
    const SeqState* __restrict__ seq, const RowNorm* __restrict__ rn,
    const double* __restrict__ lse, const float* __restrict__ gathered,
    const Cand* __restrict__ cand, const double* __restrict__ sums, int32_t* __restrict__ out_tok,
    float* __restrict__ out_prob, float* __restrict__ out_pk, float* __restrict__ out_mass) {
    constexpr int W = Loader<DT, VEC>::W;
    __shared__ Cand buf[kMergeCap];
    const int pair = blockIdx.x;
    const int G = gamma;
    const int b = pair / (G + 1);
    const int i = pair - b * (G + 1);
    const int lane = lane_id();
    const SeqState st = seq[b];
    int32_t* tok = out_tok + static_cast<size_t>(pair) * F;
    float* prob = out_prob + static_cast<size_t>(pair) * F;
    if (st.mode < 0) {
        for (int j = lane; j < F; j += 64) {
            tok[j] = -1;
            prob[j] = 0.0f;
        }
        if (lane == 0) {
            out_pk[pair] = 0.0f;
            if (out_mass)
                out_mass[pair] = 0.0f;
        }
        return;
    }

    // Probability of length i: prod_{j<i} beta_j, times (1 - beta_i) below G.
    double reach = 1.0;
    for (int j0 = 0; j0 < i; j0 += 64) {
        const int j = j0 + lane;
        const double beta = j < i ? accept_prob(j, b, G, st.mode, st.inv_t, tokens, rn, lse, gathered)
                                  : 1.0;
        reach *= wave_prod_f64(beta);
    }
    const double pk = i < G ? reach * (1.0 - accept_prob(i, b, G, st.mode, st.inv_t, tokens, rn,
                                                         lse, gathered))
                            : reach;

    // Merge the splits' lists and sums (fixed order).
    const int total = nsplit * F;
    const Cand* src = cand + static_cast<size_t>(pair) * total;
    for (int s = lane; s < total; s += 64)
        buf[s] = src[s];
    __builtin_amdgcn_wave_barrier();
    double S = 0.0;
    for (int c = 0; c < nsplit; ++c)
        S += sums[static_cast<size_t>(pair) * nsplit + c];
    WaveList L{buf, total, -__builtin_huge_valf(), kIdxNone, nullptr, 0};
    double mass = 0.0;
    if (st.mode == 1) {
        const size_t row0 = static_cast<size_t>(b) * (2 * G + 1);
        mass = i < G ? S / rn[row0 + i].s : 1.0;
        if (i < G && !(S > 0.0)) {
            // Empty residual: the extra token would be drawn from p_i; rank p'.
            RowCoefs rc = pair_coefs<DT>(draft, target, G, vocab, b, i, st, rn);
            rc.kind = kP;
            rc.qrow = rc.prow;
            L.count = 0;
            L.tv = -__builtin_huge_valf();
            L.ti = kIdxNone;
            const int groups = vocab / W;
            S = wave_sum_f64(stream_tiles<DT, VEC, false, kP, 1>(rc, groups, 0, (groups + 63) / 64,
                                                                  1, F, L));
        }
    }
    tighten<kMergeCap / 64>(L, F);
    float v;
    int idx;
    sorted_entries(L, &v, &idx);
    if (lane < F) {
        tok[lane] = idx;
        float pr = 0.0f;
        if (idx >= 0)
            pr = st.mode == 0 ? (lane == 0 ? 1.0f : 0.0f)
                              : static_cast<float>(static_cast<double>(v) / S);
        prob[lane] = pr;
    }
    if (lane == 0) {
        out_pk[pair] = static_cast<float>(pk);
        if (out_mass)
            out_mass[pair] = static_cast<float>(mass);
    }
}

template <int DT, bool VEC>
hipError_t launch_typed(const Shape& s, int nsplit, int F, const void* draft, const void* target,
                        const int32_t* tokens, const SeqState* seq, const RowNorm* rn,
                        const double* lse, const float* gathered, OutcomeWork work,
                        int32_t* out_tok, float* out_prob, float* out_pk, float* out_mass,
                        hipStream_t stream) {
    constexpr int W = Loader<DT, VEC>::W;
    const long pairs = static_cast<long>(s.batch) * (s.gamma + 1);
    const int groups = s.vocab / W;
    const int ntiles = (groups + 63) / 64;
    const int per = (ntiles + nsplit - 1) / nsplit;
    const int nsplit_eff = (ntiles + per - 1) / per;
    outcome_topf_kernel<DT, VEC, true><<<dim3(static_cast<unsigned>(pairs * nsplit_eff)),
                                         dim3(kBlock), 0, stream>>>(
        draft, target, s.gamma, s.vocab, nsplit_eff, per, F, seq, rn, work.cand, work.sums);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    outcome_merge_kernel<DT, VEC><<<dim3(static_cast<unsigned>(pairs)), dim3(64), 0, stream>>>(
        draft, target, tokens, s.gamma, s.vocab, nsplit_eff, F, seq, rn, lse, gathered, work.cand,
        work.sums, out_tok, out_prob, out_pk, out_mass);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_outcomes(const Shape& s, bool vec, int nsplit, int top_f, const void* draft,
                           const void* target, const int32_t* tokens, const SeqState* seq,
                           const RowNorm* rn, const double* lse, const float* gathered,
                           OutcomeWork work, int32_t* out_tok, float* out_prob, float* out_pk,
                           float* out_mass, hipStream_t stream) {
    if (s.batch == 0)
        return hipSuccess;
    if (s.dtype == kBF16)
        return vec ? launch_typed<kBF16, true>(s, nsplit, top_f, draft, target, tokens, seq, rn, lse,
                                               gathered, work, out_tok, out_prob, out_pk, out_mass, stream)
                   : launch_typed<kBF16, false>(s, nsplit, top_f, draft, target, tokens, seq, rn, lse,
                                                gathered, work, out_tok, out_prob, out_pk, out_mass, stream);
    return vec ? launch_typed<kF32, true>(s, nsplit, top_f, draft, target, tokens, seq, rn, lse,
                                          gathered, work, out_tok, out_prob, out_pk, out_mass, stream)
               : launch_typed<kF32, false>(s, nsplit, top_f, draft, target, tokens, seq, rn, lse,
                                           gathered, work, out_tok, out_prob, out_pk, out_mass, stream);
}

namespace {

// ----------------------------------------------------- cache budget ---
//
// One wavefront per sequence places the budget entry by entry. The lists sit
// in LDS; lane l owns lengths l, l + 64, ... (up to four) and keeps, for each,
// the key of its next unused entry and of the one after, so the lane that
// wins a step has the following key in a register while its LDS read for the
// one after that completes behind the next step. A key is the worth's binary64
// bit pattern plus one (worths are >= 0, so keys order like worths; 0 marks a
// used-up list). A step is a wavefront maximum of the lanes' best keys by DPP
// moves, then ballots for the lowest length that holds it. Worths are exact
// binary64 products, so the comparisons and the running hit sum (added in
// placement order) are reproducible bit for bit.
constexpr int kFanoutRegs = SPEC_FANOUT_MAX_LENGTHS / 64;

__device__ inline uint64_t fanout_key(float pk, float prob) {
    const double v = static_cast<double>(pk) * static_cast<double>(prob);
    return static_cast<uint64_t>(__double_as_longlong(v > 0.0 ? v : 0.0)) + 1;
}

// max(k, the key DPP pattern CTRL brings from another lane); lanes outside
// ROW_MASK, or whose source is outside the row, see 0 (below every key).
template <int CTRL, int ROW_MASK>
__device__ inline uint64_t max_dpp(uint64_t k) {
    const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(k & 0xffffffffu), CTRL, ROW_MASK,
                                               0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(k >> 32), CTRL, ROW_MASK, 0xF,
                                               false);
    const uint64_t o = (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
    return o > k ? o : k;
}

// The largest key of the wavefront, in every lane: butterflies within each
// row of 16 lanes, then the row broadcasts leave the maximum in lane 63.
__device__ inline uint64_t wave_max_key(uint64_t k) {
    k = max_dpp<0xB1, 0xF>(k);   // quad_perm [1,0,3,2]
    k = max_dpp<0x4E, 0xF>(k);   // quad_perm [2,3,0,1]
    k = max_dpp<0x141, 0xF>(k);  // row_half_mirror
    k = max_dpp<0x140, 0xF>(k);  // row_mirror: every lane holds its row's maximum
    k = max_dpp<0x142, 0xA>(k);  // row_bcast:15 into rows 1 and 3
    k = max_dpp<0x143, 0xC>(k);  // row_bcast:31 into rows 2 and 3: lane 63 = maximum
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(k & 0xffffffffu), 63));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(k >> 32), 63));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Entry by entry (any lists).
__device__ inline void fanout_sequential(int L, int F, const float* lists, const float* pk_l,
                                         int budget, int32_t* out_n, double* out_hit) {
    const int lane = threadIdx.x;
    int n[kFanoutRegs];
    float p[kFanoutRegs];
    uint64_t cur[kFanoutRegs], nxt[kFanoutRegs];  // keys of the next entry and the one after
#pragma unroll
    for (int r = 0; r < kFanoutRegs; ++r) {
        const int i = lane + 64 * r;
        n[r] = 0;
        p[r] = 0.0f;
        cur[r] = 0;
        nxt[r] = 0;
        if (i < L) {
            p[r] = pk_l[i];
            cur[r] = fanout_key(p[r], lists[i * F]);
            if (F > 1)
                nxt[r] = fanout_key(p[r], lists[i * F + 1]);
        }
    }
    double hit = 0.0;
    for (int step = 0; step < budget; ++step) {
        // The lane's best (its lowest length on equal keys), then the wavefront's.
        uint64_t best = cur[0];
        int best_r = 0;
#pragma unroll
        for (int r = 1; r < kFanoutRegs; ++r)
            if (cur[r] > best) {
                best = cur[r];
                best_r = r;
            }
        const uint64_t m = wave_max_key(best);
        if (m == 0)
            break;  // every list is used up (wave-uniform)
        // Lowest length with key m: lengths are lane + 64 r, so the lowest r
        // first, then the lowest lane.
        int win_lane = 0, win_r = 0;
#pragma unroll
        for (int r = kFanoutRegs - 1; r >= 0; --r) {
            const uint64_t sel = __ballot(best == m && best_r == r);
            if (sel) {
                win_lane = __ffsll(static_cast<long long>(sel)) - 1;
                win_r = r;
            }
        }
        hit += __longlong_as_double(static_cast<long long>(m - 1));
        if (lane == win_lane) {
#pragma unroll
            for (int r = 0; r < kFanoutRegs; ++r) {
                if (r == win_r) {
                    n[r] += 1;
                    cur[r] = nxt[r];
                    const int i = lane + 64 * r;
                    nxt[r] = n[r] + 1 < F ? fanout_key(p[r], lists[i * F + n[r] + 1]) : 0;
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < kFanoutRegs; ++r) {
        const int i = lane + 64 * r;
        if (i < L)
            out_n[i] = n[r];
    }
    if (lane == 0 && out_hit)
        *out_hit = hit;
}


// All at once, for lists whose worths do not increase along the list and at
// most kFanoutFastEntries entries: the placement above then takes the
// `budget` largest keys, the lower length and then the earlier entry first
// among equal keys, which a search over the key bits finds without stepping.
// Entry e = i F + j sits in lane e % 64, register e / 64; T is the largest
// key with at least `placed` keys >= T (one ballot count per key bit); every
// key above T is placed, and the keys equal to T are placed in entry order
// until the count is reached. Each length's placed entries are then a prefix
// of its list, counted in LDS.
constexpr int kFanoutFastRegs = 4;
constexpr int kFanoutFastEntries = 64 * kFanoutFastRegs;

__device__ inline void fanout_fast(int L, int F, const float* lists, const float* pk_l, int budget,
                                   int* counts, int32_t* out_n, double* out_hit) {
    const int lane = threadIdx.x;
    const int total = L * F;
    const int placed = budget < total ? budget : total;
    uint64_t key[kFanoutFastRegs];
#pragma unroll
    for (int k = 0; k < kFanoutFastRegs; ++k) {
        const int e = lane + 64 * k;
        key[k] = e < total ? fanout_key(pk_l[e / F], lists[e]) : 0;
    }
    auto count_ge = [&](uint64_t t) {
        int c = 0;
#pragma unroll
        for (int k = 0; k < kFanoutFastRegs; ++k)
            c += __popcll(__ballot(key[k] >= t));
        return c;
    };
    // The largest T with count_ge(T) >= placed (keys >= 1, so T >= 1 when placed >= 1).
    uint64_t t = 0;
    if (placed > 0) {
        for (int bit = 62; bit >= 0; --bit) {
            const uint64_t c = t | (1ULL << bit);
            if (count_ge(c) >= placed)
                t = c;
        }
    }
    const int above = placed > 0 ? count_ge(t + 1) : 0;
    const int ties = placed - above;  // keys equal to t to place, in entry order
    for (int i = lane; i < L; i += 64)
        counts[i] = 0;
    __syncthreads();
    double hit = 0.0;
    int before = 0;  // equal keys in earlier registers
#pragma unroll
    for (int k = 0; k < kFanoutFastRegs; ++k) {
        const int e = lane + 64 * k;
        const bool eq = placed > 0 && key[k] == t;
        const uint64_t m = __ballot(eq);
        const int rank = before + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                            __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
        before += __popcll(m);
        const bool take = e < total && placed > 0 && (key[k] > t || (eq && rank < ties));
        if (take) {
            atomicAdd(&counts[e / F], 1);
            hit += __longlong_as_double(static_cast<long long>(key[k] - 1));
        }
    }
    __syncthreads();
    for (int i = lane; i < L; i += 64)
        out_n[i] = counts[i];
    // The hit rate: lanes' partial sums added in a fixed order.
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        hit += __shfl_xor(hit, off, 64);
    if (lane == 0 && out_hit)
        *out_hit = hit;
}

__global__ __launch_bounds__(64) void outcome_fanout_kernel(int L, int F, const float* __restrict__ pk,
                                                             const float* __restrict__ probs,
                                                             int budget, int32_t* __restrict__ out_n,
                                                             double* __restrict__ out_hit) {
    extern __shared__ float lds[];  // lists [L][F], then pk [L], then counts [L]
    float* lists = lds;
    float* pk_l = lds + L * F;
    int* counts = reinterpret_cast<int*>(pk_l + L);
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const float* src = probs + static_cast<size_t>(b) * L * F;
    for (int e = lane; e < L * F; e += 64)
        lists[e] = src[e];
    for (int i = lane; i < L; i += 64)
        pk_l[i] = pk[static_cast<size_t>(b) * L + i];
    __syncthreads();
    // Do the worths fall (or stay) along every list?
    bool rising = false;
    for (int e = lane; e < L * F; e += 64)
        if (e % F != 0 && fanout_key(pk_l[e / F], lists[e]) > fanout_key(pk_l[e / F], lists[e - 1]))
            rising = true;
    int32_t* n_b = out_n + static_cast<size_t>(b) * L;
    double* hit_b = out_hit ? out_hit + b : nullptr;
    if (__ballot(rising) == 0 && L * F <= kFanoutFastEntries)
        fanout_fast(L, F, lists, pk_l, budget, counts, n_b, hit_b);
    else
        fanout_sequential(L, F, lists, pk_l, budget, n_b, hit_b);
}

bool fanout_aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace
}  // namespace specv

extern "C" int spec_outcome_fanout(int batch, int lengths, int top_f, const float* pk,
                                   const float* probs, int budget, int32_t* out_n,
                                   double* out_hit, void* hip_stream) {
    using specv::fanout_aligned;
    if (batch < 0 || lengths < 1 || lengths > SPEC_FANOUT_MAX_LENGTHS || top_f < 1 ||
        top_f > SPEC_OUTCOME_MAX_F || budget < 0)
        return SPEC_EINVAL;
    if (batch == 0)
        return SPEC_OK;
    if (!pk || !probs || !out_n || !fanout_aligned(pk, 4) || !fanout_aligned(probs, 4) ||
        !fanout_aligned(out_n, 4) || (out_hit && !fanout_aligned(out_hit, 8)))
        return SPEC_EINVAL;
    const size_t lds = (static_cast<size_t>(lengths) * top_f + 2 * lengths) * sizeof(float);
    // The largest shape needs a little over the default 64 KiB of dynamic LDS.
    static const bool lds_raised =
        hipFuncSetAttribute(reinterpret_cast<const void*>(specv::outcome_fanout_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>((SPEC_FANOUT_MAX_LENGTHS * SPEC_OUTCOME_MAX_F +
                                              2 * SPEC_FANOUT_MAX_LENGTHS) * sizeof(float))) ==
        hipSuccess;
    if (lds > 65536 && !lds_raised)
        return SPEC_EHIP;
    specv::outcome_fanout_kernel<<<dim3(static_cast<unsigned>(batch)), dim3(64), lds,
                                   static_cast<hipStream_t>(hip_stream)>>>(
        lengths, top_f, pk, probs, budget, out_n, out_hit);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

