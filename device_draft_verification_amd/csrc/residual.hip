// Residual / bonus kernel: draws the extra token of every sampled sequence.
//
// At the first rejected position k < G the token comes from the residual
// r_v = max(0, p_k(v) - q_k(v)); when all G drafts were kept it is the bonus
// token, r_v = p_G(v) (Speculative Speculative Decoding summary, section 2,
// Saguaro challenge 2: the residual distribution is what the bonus token is
// sampled from). The draw inverts u_res * S on the prefix sums of r in
// vocabulary order: the token is the first v whose inclusive prefix exceeds
// u_res * S, S = sum_v r_v.
//
// Work layout: grid = B * nsplit workgroups; workgroup (b, c) streams split c
// of the one or two rows of sequence b and publishes the split's sum of r.
// An agent-scope ticket elects the last workgroup of the sequence, which scans
// the split sums in order, finds the split holding u_res * S and re-reads only
// that split, in index order, to find the token. Atomics choose who finishes,
// never the order of any sum, so the result is bitwise reproducible.
//
// p and q are recomputed from the row normalisers of the row kernel:
// p_v = 2^(fma(x_v, log2e, -m)) / s, which sums to one under the same
// normaliser the accept test used. r is formed in fp32 and accumulated in fp64.
#include "launch.hpp"

namespace specv {
namespace {

struct RowCoef {
    float m;     // base-2 reference of the row
    float inv_s; // 1 / s
};

template <int DT, bool VEC>
__device__ inline void residual_group(const void* prow, const void* qrow, bool p_only,
                                      float inv_t, RowCoef cp, RowCoef cq, long g,
                                      float (&r)[Group<DT, VEC>::W]) {
    using Ld = Loader<DT, VEC>;
    constexpr int W = Ld::W;
    float zp[W];
    Ld::unpack(Ld::load(prow, g), zp);
    if (p_only) {
#pragma unroll
        for (int e = 0; e < W; ++e)
            r[e] = fast_exp2(__builtin_fmaf(scale_logit(zp[e], inv_t), kLog2e, -cp.m)) * cp.inv_s;
        return;
    }
    float zq[W];
    Ld::unpack(Ld::load(qrow, g), zq);
#pragma unroll
    for (int e = 0; e < W; ++e) {
        const float p = fast_exp2(__builtin_fmaf(scale_logit(zp[e], inv_t), kLog2e, -cp.m)) * cp.inv_s;
        const float q = fast_exp2(__builtin_fmaf(scale_logit(zq[e], inv_t), kLog2e, -cq.m)) * cq.inv_s;
        r[e] = fmaxf(p - q, 0.0f);
    }
}

// Sum of r over groups [g0, g1) with a kBlock-strided, U-deep load pattern.
template <int DT, bool VEC, int U>
__device__ inline double range_sum(const void* prow, const void* qrow, bool p_only, float inv_t,
                                   RowCoef cp, RowCoef cq, long g0, long g1, double* lds_d) {
    constexpr int W = Group<DT, VEC>::W;
    double acc = 0.0;
    long g = g0 + threadIdx.x;
    for (; g + static_cast<long>(U - 1) * kBlock < g1; g += static_cast<long>(U) * kBlock) {
        float r[U][W];
#pragma unroll
        for (int u = 0; u < U; ++u)
            residual_group<DT, VEC>(prow, qrow, p_only, inv_t, cp, cq, g + static_cast<long>(u) * kBlock, r[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float t = 0.0f;
#pragma unroll
            for (int e = 0; e < W; ++e)
                t += r[u][e];
            acc += static_cast<double>(t);
        }
    }
    for (; g < g1; g += kBlock) {
        float r[W];
        residual_group<DT, VEC>(prow, qrow, p_only, inv_t, cp, cq, g, r);
        float t = 0.0f;
#pragma unroll
        for (int e = 0; e < W; ++e)
            t += r[e];
        acc += static_cast<double>(t);
    }
    return block_sum(acc, lds_d);
}

struct ScanLds {
    double d[kWaves];
    int i[kWaves];
    int result;
};

// First element v of groups [g0, g1) (index order) at which P + prefix(r)
// exceeds tau, with r_v > 0. Each thread takes kGpt consecutive groups, the
// block scans the per-thread sums, and the thread holding the crossing walks
// its elements. When the range ends first (possible only through rounding at
// its last edge) returns -2 - (last element with r > 0), which is <= -2.
template <int DT, bool VEC>
__device__ int scan_range(const void* prow, const void* qrow, bool p_only, float inv_t,
                          RowCoef cp, RowCoef cq, long g0, long g1, double P, double tau,
                          ScanLds& lds) {
    constexpr int W = Group<DT, VEC>::W;
    constexpr int kGpt = VEC ? 4 : 16;
    int last_pos = -1;
    for (long base = g0; base < g1; base += static_cast<long>(kBlock) * kGpt) {
        const long my0 = base + static_cast<long>(threadIdx.x) * kGpt;
        float r[kGpt][W];
#pragma unroll
        for (int q = 0; q < kGpt; ++q) {
            if (my0 + q < g1) {
                residual_group<DT, VEC>(prow, qrow, p_only, inv_t, cp, cq, my0 + q, r[q]);
            } else {
#pragma unroll
                for (int e = 0; e < W; ++e)
                    r[q][e] = 0.0f;
            }
        }
        double mine = 0.0;
        int my_last = -1;
#pragma unroll
        for (int q = 0; q < kGpt; ++q) {
#pragma unroll
            for (int e = 0; e < W; ++e) {
                mine += static_cast<double>(r[q][e]);
                if (r[q][e] > 0.0f)
                    my_last = static_cast<int>((my0 + q) * W + e);
            }
        }
        double total;
        const double excl = block_exclusive_scan(mine, lds.d, &total);
        double a = P + excl;
        int hit = -1;
#pragma unroll
        for (int q = 0; q < kGpt; ++q) {
#pragma unroll
            for (int e = 0; e < W; ++e) {
                a += static_cast<double>(r[q][e]);
                if (hit < 0 && r[q][e] > 0.0f && a > tau)
                    hit = static_cast<int>((my0 + q) * W + e);
            }
        }
        const int first = block_first(hit >= 0, lds.i);
        if (first < kBlock) {
            if (static_cast<int>(threadIdx.x) == first)
                lds.result = hit;
            __syncthreads();
            return lds.result;
        }
        const int lp = block_max_int(my_last, lds.i);
        last_pos = lp > last_pos ? lp : last_pos;
        P = P + total;
    }
    return -2 - last_pos;
}

template <int DT, bool VEC, int U>
__global__ __launch_bounds__(kBlock) void residual_kernel(
    const void* __restrict__ draft, const void* __restrict__ target,
    const float* __restrict__ temperature, int gamma, int vocab, int nsplit,
    const SeqState* __restrict__ seq, const RowNorm* __restrict__ rn,
    double* __restrict__ chunk_sums, int* __restrict__ tickets, int32_t* __restrict__ out_tok) {
    constexpr int W = Group<DT, VEC>::W;
    const long blk = blockIdx.x;
    const int c = static_cast<int>(blk % nsplit);
    const long b = blk / nsplit;
    const SeqState st = seq[b];
    if (st.mode != 1)
        return;  // greedy or rejected sequence: nothing to draw
    const int G = gamma;
    const int k = st.k;
    float inv_t = 0.0f;
    temperature_mode(temperature[b], &inv_t);
    const bool bonus = k == G;
    const size_t row0 = static_cast<size_t>(b) * (2 * G + 1);
    const void* prow = row_ptr(target, DT, static_cast<size_t>(b) * (G + 1) + k, vocab);
    const void* qrow = bonus ? prow : row_ptr(draft, DT, static_cast<size_t>(b) * G + k, vocab);
    const RowNorm np = rn[row0 + G + k];
    const RowCoef cp{np.m, static_cast<float>(1.0 / np.s)};
    RowCoef cq{0.0f, 0.0f};
    if (!bonus) {
        const RowNorm nq = rn[row0 + k];
        cq = RowCoef{nq.m, static_cast<float>(1.0 / nq.s)};
    }

    __shared__ double lds_d[kWaves];
    __shared__ ScanLds scan_lds;
    __shared__ double s_sums[kMaxSplit];
    __shared__ int s_last;
    __shared__ double s_P, s_tau;
    __shared__ int s_cstar, s_fallback;

    const long groups = vocab / W;
    long g0, g1;
    split_range(groups, nsplit, c, &g0, &g1);
    const double mine = range_sum<DT, VEC, U>(prow, qrow, bonus, inv_t, cp, cq, g0, g1, lds_d);

    if (threadIdx.x == 0) {
        chunk_sums[b * nsplit + c] = mine;
        const int before = __hip_atomic_fetch_add(&tickets[b], 1, __ATOMIC_ACQ_REL,
                                                  __HIP_MEMORY_SCOPE_AGENT);
        s_last = before == nsplit - 1;
    }
    __syncthreads();
    if (!s_last)
        return;

    // The last workgroup of sequence b: locate the split, then the token.
    if (threadIdx.x == 0) {
        double S = 0.0;
        for (int cc = 0; cc < nsplit; ++cc) {
            s_sums[cc] = __hip_atomic_load(&chunk_sums[b * nsplit + cc], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
            S += s_sums[cc];
        }
        __hip_atomic_store(&tickets[b], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (S > 0.0) {
            const double tau = static_cast<double>(st.u_res) * S;
            double P = 0.0;
            int cstar = nsplit - 1;
            for (int cc = 0; cc < nsplit; ++cc) {
                if (P + s_sums[cc] > tau) {
                    cstar = cc;
                    break;
                }
                P += s_sums[cc];
            }
            s_P = P;
            s_tau = tau;
            s_cstar = cstar;
            s_fallback = 0;
        } else {
            s_fallback = 1;
        }
    }
    __syncthreads();

    int token;
    if (!s_fallback) {
        long c0, c1;
        split_range(groups, nsplit, s_cstar, &c0, &c1);
        token = scan_range<DT, VEC>(prow, qrow, bonus, inv_t, cp, cq, c0, c1, s_P, s_tau, scan_lds);
    } else {
        // Empty residual (possible only through rounding when p and q agree
        // to within fp32): draw from p at the same position instead.
        const double Sp = range_sum<DT, VEC, U>(prow, prow, true, inv_t, cp, cp, 0, groups, lds_d);
        const double tau = static_cast<double>(st.u_res) * Sp;
        token = scan_range<DT, VEC>(prow, prow, true, inv_t, cp, cp, 0, groups, 0.0, tau, scan_lds);
    }
    if (token <= -2)
        token = -2 - token;  // the range ended first: its last positive element
    if (threadIdx.x == 0)
        out_tok[b * (G + 1) + k] = token;
}

template <int DT, bool VEC>
hipError_t launch_typed(const Shape& sh, int nsplit, const void* draft, const void* target,
                        const float* temperature, const SeqState* seq, const RowNorm* rn,
                        double* chunk_sums, int* tickets, int32_t* out_tok, hipStream_t stream) {
    constexpr int U = VEC ? 2 : 8;
    const long blocks = static_cast<long>(sh.batch) * nsplit;
    if (blocks == 0)
        return hipSuccess;
    residual_kernel<DT, VEC, U><<<dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, stream>>>(
        draft, target, temperature, sh.gamma, sh.vocab, nsplit, seq, rn, chunk_sums, tickets, out_tok);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_residual(const Shape& s, bool vec, int nsplit, const void* draft,
                           const void* target, const float* temperature, const SeqState* seq,
                           const RowNorm* rn, double* chunk_sums, int* tickets,
                           int32_t* out_tok, hipStream_t stream) {
    if (nsplit < 1 || nsplit > kMaxSplit)
        return hipErrorInvalidValue;
    if (s.dtype == kBF16)
        return vec ? launch_typed<kBF16, true>(s, nsplit, draft, target, temperature, seq, rn,
                                               chunk_sums, tickets, out_tok, stream)
                   : launch_typed<kBF16, false>(s, nsplit, draft, target, temperature, seq, rn,
                                                chunk_sums, tickets, out_tok, stream);
    return vec ? launch_typed<kF32, true>(s, nsplit, draft, target, temperature, seq, rn, chunk_sums,
                                          tickets, out_tok, stream)
               : launch_typed<kF32, false>(s, nsplit, draft, target, temperature, seq, rn,
                                           chunk_sums, tickets, out_tok, stream);
}

}  // namespace specv
