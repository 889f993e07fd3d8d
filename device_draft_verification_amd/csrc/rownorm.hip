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

// Adds a batch of N scaled logits to the running (m, s), moving the reference m
// to the batch max first: max(m, fl32(max x * log2e)).
template <int N>
__device__ inline void online_add(const float (&x)[N], float& m, double& s) {
    float gm = x[0];
#pragma unroll
    for (int e = 1; e < N; ++e)
        gm = fmaxf(gm, x[e]);
    const float mn = fmaxf(m, gm * kLog2e);
    float t[N];
#pragma unroll
    for (int e = 0; e < N; ++e)
        t[e] = fast_exp2(__builtin_fmaf(x[e], kLog2e, -mn));
    const float g = pairwise_sum(t);
    const float sc = (mn == m) ? 1.0f : fast_exp2(m - mn);
    s = __builtin_fma(s, static_cast<double>(sc), static_cast<double>(g));
    m = mn;
}

// The same with a lazy reference: the batch is summed against the current m,
// and only a batch whose sum leaves [0, 2^64] (a term above 2^64: the
// reference is far below the batch max, or no finite reference yet) is redone
// with online_add. Terms up to 2^64 are exact in fp32 range, so the result is
// a valid (m, s) pair; m may sit below the row max by up to 64 in base-2 units.
template <int N>
__device__ inline void lazy_add(const float (&x)[N], float& m, double& s) {
    float t[N];
#pragma unroll
    for (int e = 0; e < N; ++e)
        t[e] = fast_exp2(__builtin_fmaf(x[e], kLog2e, -m));
    const float g = pairwise_sum(t);
    if (g <= 18446744073709551616.0f) {
        s += static_cast<double>(g);
        return;
    }
    online_add(x, m, s);
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

    const long groups = vocab / W;
    long g0, g1;
    split_range(groups, nsplit, c, &g0, &g1);

    __shared__ float lds_f[kWaves];
    __shared__ double lds_d[kWaves];
    __shared__ int lds_i[kWaves];

    if (mode == 0) {
        // Greedy row: largest raw logit, lowest index on ties. Each thread
        // visits its indices in increasing order, so a strict '>' keeps the
        // lowest index of equal values.
        float bv = -__builtin_huge_valf();
        int bi = 0x7fffffff;
        for (long g = g0 + threadIdx.x; g < g1; g += static_cast<long>(U) * kBlock) {
            typename Ld::raw_t q[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const long idx = g + static_cast<long>(u) * kBlock;
                q[u] = idx < g1 ? Ld::template load_as<NT>(rp, idx) : Ld::neg_inf();
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float z[W];
                Ld::unpack(q[u], z);
#pragma unroll
                for (int e = 0; e < W; ++e) {
                    if (z[e] > bv) {
                        bv = z[e];
                        bi = static_cast<int>((g + static_cast<long>(u) * kBlock) * W + e);
                    }
                }
            }
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

    // The draft token scored by this row (rows of position i < G): the thread
    // whose batch holds its group records the raw logit for the accept kernel,
    // which then needs no gather of its own.
    const int pos = is_draft ? j : j - gamma;
    long tg = -1;
    int te = 0;
    if (pos < gamma) {
        const int t = tokens[static_cast<size_t>(b) * gamma + pos];
        if (t >= 0 && t < vocab) {
            tg = t / W;
            te = t % W;
        }
    }

    // Every batch is U groups wide; groups past the split's end read as -inf,
    // which adds nothing, so the split's tail keeps U loads in flight too.
    float m = kNegMax;
    double s = 0.0;
    bool first = true;
    for (long g = g0 + threadIdx.x; g < g1; g += static_cast<long>(U) * kBlock) {
        typename Ld::raw_t q[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const long idx = g + static_cast<long>(u) * kBlock;
            q[u] = idx < g1 ? Ld::template load_as<NT>(rp, idx) : Ld::neg_inf();
        }
        // (only inside this split: groups past g1 were not loaded here)
        if (tg >= g && tg < g1 && tg < g + static_cast<long>(U) * kBlock && (tg - g) % kBlock == 0) {
            const int uu = static_cast<int>((tg - g) / kBlock);
            float zt = 0.0f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float z[W];
                Ld::unpack(q[u], z);
#pragma unroll
                for (int e = 0; e < W; ++e)
                    zt = (u == uu && e == te) ? z[e] : zt;
            }
            gathered[row] = zt;
        }
        float x[U * W];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float z[W];
            Ld::unpack(q[u], z);
#pragma unroll
            for (int e = 0; e < W; ++e)
                x[u * W + e] = scale_logit(z[e], inv_t);
        }
        // the first batch sets the reference; later batches rarely move it
        if (first) {
            online_add(x, m, s);
            first = false;
        } else {
            lazy_add(x, m, s);
        }
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
                        float* gathered, hipStream_t stream) {
    const long rows = static_cast<long>(sh.batch) * (2 * sh.gamma + 1);
    const long blocks = rows * nsplit;
    if (blocks == 0)
        return hipSuccess;
    row_norm_kernel<DT, VEC, U, NT><<<dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, stream>>>(
        draft, target, temperature, tokens, sh.gamma, sh.vocab, nsplit, part, gathered);
    return hipGetLastError();
}

template <int DT, bool VEC>
hipError_t launch_unroll(const Shape& sh, const RowTuning& tu, const void* draft,
                         const void* target, const float* temperature, const int32_t* tokens,
                         Partial* part, float* gathered, hipStream_t stream) {
    if constexpr (!VEC) {
        return launch_typed<DT, false, 8, false>(sh, tu.nsplit, draft, target, temperature, tokens, part, gathered, stream);
    } else {
        if (tu.nontemporal) {
            switch (tu.unroll) {
            case 2: return launch_typed<DT, true, 2, true>(sh, tu.nsplit, draft, target, temperature, tokens, part, gathered, stream);
            case 8: return launch_typed<DT, true, 8, true>(sh, tu.nsplit, draft, target, temperature, tokens, part, gathered, stream);
            default: return launch_typed<DT, true, 4, true>(sh, tu.nsplit, draft, target, temperature, tokens, part, gathered, stream);
            }
        }
        switch (tu.unroll) {
        case 2: return launch_typed<DT, true, 2, false>(sh, tu.nsplit, draft, target, temperature, tokens, part, gathered, stream);
        case 8: return launch_typed<DT, true, 8, false>(sh, tu.nsplit, draft, target, temperature, tokens, part, gathered, stream);
        default: return launch_typed<DT, true, 4, false>(sh, tu.nsplit, draft, target, temperature, tokens, part, gathered, stream);
        }
    }
}

}  // namespace

hipError_t launch_row_norm(const Shape& s, bool vec, const RowTuning& tu, const void* draft,
                           const void* target, const float* temperature, const int32_t* tokens,
                           Partial* part, float* gathered, hipStream_t stream) {
    if (s.dtype == kBF16)
        return vec ? launch_unroll<kBF16, true>(s, tu, draft, target, temperature, tokens, part, gathered, stream)
                   : launch_unroll<kBF16, false>(s, tu, draft, target, temperature, tokens, part, gathered, stream);
    return vec ? launch_unroll<kF32, true>(s, tu, draft, target, temperature, tokens, part, gathered, stream)
               : launch_unroll<kF32, false>(s, tu, draft, target, temperature, tokens, part, gathered, stream);
}

}  // namespace specv
