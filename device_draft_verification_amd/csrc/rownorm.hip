// Row normaliser kernel: temperature scaling, then a single-pass online
// max / log-sum-exp over the vocabulary of every draft and target row (sampled
// sequences), or the raw-logit argmax of every target row (greedy sequences).
//
// This is the step that touches O(B * gamma * V) bytes: the FlashSpec summary
// (Problem statement item 1; Methodology section 1, complexity bullet) puts
// the cost of verification in this traffic and in the host sync that grows
// with V. Temperature is applied before the normaliser (same section,
// numerical-stability bullet).
//
// Layout of the work: workgroup w handles split c = w % nsplit of row
// w / nsplit; row r of sequence b = r / (2G+1) is draft row j = r % (2G+1) when
// j < G, else target row j - G. Each thread streams 16-byte groups (8 bf16 or
// 4 fp32) at a stride of kBlock groups, U groups in flight, so every load
// instruction of a wavefront reads 1 KiB of consecutive memory.
//
// Numerics: x = fl32(z * fl32(1/T)). A thread keeps a base-2 reference m and
// an fp64 sum s = sum 2^(x * log2e - m). Its first batch of U groups sets m to
// fl32(max x * log2e); each later batch adds sum_e 2^(fma(x_e, log2e, -m)),
// summed pairwise in fp32, and only when that sum exceeds 2^64 (a term far
// above the reference) moves m to the batch max, rescaling s by 2^(m_old -
// m_new). Threads are merged by rescaling each to the block's largest m once
// and adding in fp64 in a fixed tree, so the result is bitwise reproducible.
#include "launch.hpp"

namespace specv {
namespace {

template <int N>
__device__ inline float pairwise_sum(float (&t)[N]) {
#pragma unroll
    for (int w = 1; w < N; w <<= 1) {
#pragma unroll
        for (int i = 0; i + w < N; i += 2 * w)
            t[i] += t[i + w];
    }
    return t[0];
}

// Batch helpers on the raw loads of U groups (W logits each). Sums are formed
// per group by a pairwise tree and then by a pairwise tree over the groups,
// i.e. a pairwise tree over the batch in index-within-batch order.

// Largest scaled logit of the batch.
template <class Ld, int U>
__device__ inline float batch_max(const typename Ld::raw_t (&q)[U], float inv_t) {
    float gm = -__builtin_huge_valf();
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float z[Ld::W];
        Ld::unpack(q[u], z);
#pragma unroll
        for (int e = 0; e < Ld::W; ++e)
            gm = fmaxf(gm, scale_logit(z[e], inv_t));
    }
    return gm;
}

// sum over the batch of 2^(fma(x, log2e, -m)), x = fl32(z * inv_t)
template <class Ld, int U>
__device__ inline float batch_sum(const typename Ld::raw_t (&q)[U], float inv_t, float m) {
    float gs[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float z[Ld::W];
        Ld::unpack(q[u], z);
        float t[Ld::W];
#pragma unroll
        for (int e = 0; e < Ld::W; ++e)
            t[e] = fast_exp2(__builtin_fmaf(scale_logit(z[e], inv_t), kLog2e, -m));
        gs[u] = pairwise_sum(t);
    }
    return pairwise_sum(gs);
}

// Adds a batch to the running (m, s), first moving the reference m to
// max(m, fl32(batch max * log2e)) and rescaling s by 2^(m_old - m_new).
template <class Ld, int U>
__device__ inline void online_add(const typename Ld::raw_t (&q)[U], float inv_t, float& m,
                                  double& s) {
    const float mn = fmaxf(m, batch_max<Ld, U>(q, inv_t) * kLog2e);
    const float g = batch_sum<Ld, U>(q, inv_t, mn);
    const float sc = (mn == m) ? 1.0f : fast_exp2(m - mn);
    s = __builtin_fma(s, static_cast<double>(sc), static_cast<double>(g));
    m = mn;
}

// The same with a lazy reference: the batch is summed against the current m,
// and only a batch whose sum leaves [0, 2^64] (a term above 2^64: the
// reference is far below the batch max, or there is no finite reference yet)
// is redone with online_add. Terms up to 2^64 are well inside the fp32 range,
// so the result is a valid (m, s) pair; m may sit below the row max by up to
// 64 in base-2 units.
template <class Ld, int U>
__device__ inline void lazy_add(const typename Ld::raw_t (&q)[U], float inv_t, float& m,
                                double& s) {
    const float g = batch_sum<Ld, U>(q, inv_t, m);
    if (g <= 18446744073709551616.0f) {
        s += static_cast<double>(g);
        return;
    }
    online_add<Ld, U>(q, inv_t, m, s);
}

template <int DT, bool VEC, int U, bool NT>
__global__ __launch_bounds__(kBlock) void row_norm_kernel(
    const void* __restrict__ draft, const void* __restrict__ target,
    const float* __restrict__ temperature, const int32_t* __restrict__ tokens, int gamma,
    int vocab, int nsplit, Partial* __restrict__ part, float* __restrict__ gathered) {
    using Ld = Loader<DT, VEC>;
    constexpr int W = Ld::W;
    const long blk = blockIdx.x;
    const int c = static_cast<int>(blk % nsplit);
    const long row = blk / nsplit;
    const int rps = 2 * gamma + 1;
    const long b = row / rps;
    const int j = static_cast<int>(row % rps);

    float inv_t = 0.0f;
    const int mode = temperature_mode(temperature[b], &inv_t);
    const bool is_draft = j < gamma;
    if (mode < 0 || (mode == 0 && is_draft))
        return;  // nothing of this row is used
    const void* rp = is_draft
        ? row_ptr(draft, DT, static_cast<size_t>(b) * gamma + j, vocab)
        : row_ptr(target, DT, static_cast<size_t>(b) * (gamma + 1) + (j - gamma), vocab);

    // Splits are whole multiples of a batch stride (U groups per thread), so
    // only the row's last split ends in a partial batch.
    const int groups = vocab / W;
    constexpr int kStride = U * kBlock;
    const int strides = (groups + kStride - 1) / kStride;
    const int per = (strides + nsplit - 1) / nsplit * kStride;
    const int g0 = c * per < groups ? c * per : groups;
    const int g1 = g0 + per < groups ? g0 + per : groups;
    // g < full_end: all U groups of the batch lie inside the split
    const int full_end = g1 - (U - 1) * kBlock;

    __shared__ float lds_f[kWaves];
    __shared__ double lds_d[kWaves];
    __shared__ int lds_i[kWaves];

    auto load_batch = [&](int g, typename Ld::raw_t (&q)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            q[u] = Ld::template load_as<NT>(rp, g + u * kBlock);
    };
    auto load_batch_tail = [&](int g, typename Ld::raw_t (&q)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = g + u * kBlock;
            q[u] = idx < g1 ? Ld::template load_as<NT>(rp, idx) : Ld::neg_inf();
        }
    };

    if (mode == 0) {
        // Greedy row: largest raw logit, lowest index on ties. Each thread
        // visits its indices in increasing order, so a strict '>' keeps the
        // lowest index of equal values.
        float bv = -__builtin_huge_valf();
        int bi = 0x7fffffff;
        auto scan = [&](int g, const typename Ld::raw_t (&q)[U]) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float z[W];
                Ld::unpack(q[u], z);
#pragma unroll
                for (int e = 0; e < W; ++e) {
                    if (z[e] > bv) {
                        bv = z[e];
                        bi = (g + u * kBlock) * W + e;
                    }
                }
            }
        };
        int g = g0 + threadIdx.x;
        for (; g < full_end; g += U * kBlock) {
            typename Ld::raw_t q[U];
            load_batch(g, q);
            scan(g, q);
        }
        if (g < g1) {
            typename Ld::raw_t q[U];
            load_batch_tail(g, q);
            scan(g, q);
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off, 64);
            const int oi = __shfl_xor(bi, off, 64);
            if (ov > bv || (ov == bv && oi < bi)) {
                bv = ov;
                bi = oi;
            }
        }
        const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
        if (lane == 0) {
            lds_f[wid] = bv;
            lds_i[wid] = bi;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int w = 1; w < kWaves; ++w) {
                if (lds_f[w] > bv || (lds_f[w] == bv && lds_i[w] < bi)) {
                    bv = lds_f[w];
                    bi = lds_i[w];
                }
            }
            part[blk] = Partial{bv, bi, 0.0};
        }
        return;
    }

    // The draft token scored by this row (rows of position i < G): the one
    // thread whose groups include the token's group records its raw logit for
    // the accept kernel, which then needs no gather of its own. Thread t visits
    // groups g0 + t + n * kBlock, n = 0, 1, ..., in batches of U.
    const int pos = is_draft ? j : j - gamma;
    int cap_batch = -1, cap_u = 0, cap_e = 0;
    if (pos < gamma) {
        const int t = tokens[static_cast<size_t>(b) * gamma + pos];
        if (t >= 0 && t < vocab) {
            const int tg = t / W;
            if (tg >= g0 && tg < g1 && (tg - g0) % kBlock == static_cast<int>(threadIdx.x)) {
                const int n = (tg - g0) / kBlock;
                cap_batch = n / U;
                cap_u = n % U;
                cap_e = t % W;
            }
        }
    }
    auto capture = [&](const typename Ld::raw_t (&q)[U]) {
        float zt = 0.0f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float z[W];
            Ld::unpack(q[u], z);
#pragma unroll
            for (int e = 0; e < W; ++e)
                zt = (u == cap_u && e == cap_e) ? z[e] : zt;
        }
        gathered[row] = zt;
    };

    // (m, s) accumulation. Full batches load without predication; the split's
    // last partial batch reads groups past its end as -inf, which adds nothing.
    float m = kNegMax;
    double s = 0.0;
    auto accumulate = [&](const typename Ld::raw_t (&q)[U], bool first) {
        // the first batch sets the reference; later batches rarely move it
        if (first)
            online_add<Ld, U>(q, inv_t, m, s);
        else
            lazy_add<Ld, U>(q, inv_t, m, s);
    };
    int g = g0 + threadIdx.x;
    int batch = 0;
    for (; g < full_end; g += U * kBlock, ++batch) {
        typename Ld::raw_t q[U];
        load_batch(g, q);
        if (batch == cap_batch)
            capture(q);
        accumulate(q, batch == 0);
    }
    if (g < g1) {
        typename Ld::raw_t q[U];
        load_batch_tail(g, q);
        if (batch == cap_batch)
            capture(q);
        accumulate(q, batch == 0);
    }

    const float bm = block_max(m, lds_f);
    const float sc = (m == bm) ? 1.0f : fast_exp2(m - bm);
    const double bs = block_sum(s * static_cast<double>(sc), lds_d);
    if (threadIdx.x == 0)
        part[blk] = Partial{bm, -1, bs};
}

template <int DT, bool VEC, int U, bool NT>
hipError_t launch_typed(const Shape& sh, int nsplit, const void* draft, const void* target,
                        const float* temperature, const int32_t* tokens, Partial* part,
                        float* gathered, hipStream_t stream, const LaunchEvents& ev) {
    const long rows = static_cast<long>(sh.batch) * (2 * sh.gamma + 1);
    const long blocks = rows * nsplit;
    if (blocks == 0)
        return hipSuccess;
    return launch(row_norm_kernel<DT, VEC, U, NT>, dim3(static_cast<unsigned>(blocks)),
                  dim3(kBlock), 0, stream, ev, draft, target, temperature, tokens, sh.gamma,
                  sh.vocab, nsplit, part, gathered);
}

template <int DT, bool VEC>
hipError_t launch_unroll(const Shape& sh, const RowTuning& tu, const void* draft,
                         const void* target, const float* temperature, const int32_t* tokens,
                         Partial* part, float* gathered, hipStream_t stream,
                         const LaunchEvents& ev) {
    if constexpr (!VEC) {
        return launch_typed<DT, false, 8, false>(sh, tu.nsplit, draft, target, temperature, tokens, part, gathered, stream, ev);
    } else {
        if (tu.nontemporal) {
            switch (tu.unroll) {
            case 2: return launch_typed<DT, true, 2, true>(sh, tu.nsplit, draft, target, temperature, tokens, part, gathered, stream, ev);
            case 8: return launch_typed<DT, true, 8, true>(sh, tu.nsplit, draft, target, temperature, tokens, part, gathered, stream, ev);
            default: return launch_typed<DT, true, 4, true>(sh, tu.nsplit, draft, target, temperature, tokens, part, gathered, stream, ev);
            }
        }
        switch (tu.unroll) {
        case 2: return launch_typed<DT, true, 2, false>(sh, tu.nsplit, draft, target, temperature, tokens, part, gathered, stream, ev);
        case 8: return launch_typed<DT, true, 8, false>(sh, tu.nsplit, draft, target, temperature, tokens, part, gathered, stream, ev);
        default: return launch_typed<DT, true, 4, false>(sh, tu.nsplit, draft, target, temperature, tokens, part, gathered, stream, ev);
        }
    }
}

}  // namespace

hipError_t launch_row_norm(const Shape& s, bool vec, const RowTuning& tu, const void* draft,
                           const void* target, const float* temperature, const int32_t* tokens,
                           Partial* part, float* gathered, hipStream_t stream,
                           const LaunchEvents& ev) {
    if (s.dtype == kBF16)
        return vec ? launch_unroll<kBF16, true>(s, tu, draft, target, temperature, tokens, part, gathered, stream, ev)
                   : launch_unroll<kBF16, false>(s, tu, draft, target, temperature, tokens, part, gathered, stream, ev);
    return vec ? launch_unroll<kF32, true>(s, tu, draft, target, temperature, tokens, part, gathered, stream, ev)
               : launch_unroll<kF32, false>(s, tu, draft, target, temperature, tokens, part, gathered, stream, ev);
}

}  // namespace specv
