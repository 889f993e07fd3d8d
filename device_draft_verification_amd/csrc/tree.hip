// Draft trees: confidence-guided pruning and greedy tree verification.
//
// Pruning (SpecLA summary, Methodology section 3): a tree's low-probability
// paths are cut by their cumulative draft log-probability before the target
// verifies them. One workgroup per tree, one thread per node (M <= 256; up to
// 64 nodes one wavefront, with shuffles in place of the barriers):
//   * path scores c(i) = c(parent) + logq(i) are resolved level by level, each
//     with the one double addition the definition states, so they equal the
//     root-down sums bit for bit;
//   * a node's rank is the number of nodes with a larger score (ties to the
//     lower index), counted over the scores in LDS;
//   * kept nodes (score >= tau, rank < budget) are renumbered by a ballot
//     prefix count, and their parents remapped.
// Greedy verification (T = 0, the exact-match rule of token-tree decoding):
//   tree_argmax_kernel: the raw-logit argmax of every node's target row, split
//     over the vocabulary like the row normaliser (16-byte loads);
//   tree_walk_kernel: one wavefront per tree merges the splits of the rows it
//     reaches and walks from the root to the lowest-index child whose token is
//     the argmax, with one ballot per 64 candidate children.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <new>

#include "launch.hpp"
#include "spec_tree.h"

namespace specv {
namespace {

constexpr int kTreeThreads = SPEC_TREE_MAX_NODES;  // one thread per node

__global__ __launch_bounds__(kTreeThreads) void tree_prune_kernel(
    const int32_t* __restrict__ parent, const float* __restrict__ logq, int M, double tau,
    int budget, double* __restrict__ cum, int32_t* __restrict__ new_index,
    int32_t* __restrict__ new_parent, int32_t* __restrict__ count) {
    __shared__ double c[kTreeThreads];
    __shared__ int par[kTreeThreads];
    __shared__ int ready[kTreeThreads];
    __shared__ int ni[kTreeThreads];
    __shared__ int old_of_new[kTreeThreads];
    __shared__ int wave_kept[kTreeThreads / 64];
    const int b = blockIdx.x, i = threadIdx.x;
    const int lane = i & 63, w = i >> 6;
    const bool node = i < M;
    const size_t base = static_cast<size_t>(b) * M;
    const int p = node ? parent[base + i] : -1;
    const float lq = node ? logq[base + i] : 0.0f;
    const bool bad = node && (i == 0 ? p != -1 : (p < 0 || p >= i || !(lq <= 0.0f)));
    if (__syncthreads_or(bad)) {
        if (node) {
            cum[base + i] = __builtin_nan("");
            new_index[base + i] = -1;
            new_parent[base + i] = -1;
        }
        if (i == 0)
            count[b] = -1;
        return;
    }
    par[i] = p;
    c[i] = 0.0;
    ready[i] = i == 0 || !node;
    __syncthreads();
    // One tree level per round: a node whose parent is final adds its own term.
    for (;;) {
        const bool waiting = !ready[i];
        if (!__syncthreads_or(waiting))
            break;
        bool done = false;
        if (waiting && ready[p]) {
            c[i] = c[p] + static_cast<double>(lq);
            done = true;
        }
        __syncthreads();
        if (done)
            ready[i] = 1;
        __syncthreads();
    }
    int rank = 0;
    if (node) {
        const double ci = c[i];
        for (int j = 0; j < M; ++j) {
            const double cj = c[j];
            rank += (cj > ci || (cj == ci && j < i)) ? 1 : 0;
        }
    }
    const bool keep = node && c[i] >= tau && rank < budget;
    const unsigned long long m = __ballot(keep);
    if (lane == 0)
        wave_kept[w] = __popcll(m);
    __syncthreads();
    int before = __builtin_amdgcn_mbcnt_hi(static_cast<unsigned>(m >> 32),
                                           __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(m), 0));
    int total = 0;
    for (int v = 0; v < kTreeThreads / 64; ++v) {
        if (v < w)
            before += wave_kept[v];
        total += wave_kept[v];
    }
    ni[i] = keep ? before : -1;
    if (keep)
        old_of_new[before] = i;
    __syncthreads();
    if (node) {
        cum[base + i] = c[i];
        new_index[base + i] = ni[i];
        int np = -1;
        if (i < total) {
            const int old = old_of_new[i];
            np = old == 0 ? -1 : ni[par[old]];
        }
        new_parent[base + i] = np;
    }
    if (i == 0)
        count[b] = total;
}

// Trees of at most 64 nodes: one wavefront per tree, node i on lane i, the
// same three steps without a barrier. Path scores resolve level by level
// through lane shuffles (a node adds its own term once, to its parent's final
// score, so the sums are the root-down ones bit for bit); a node's rank counts
// the scores broadcast lane by lane; the kept nodes are renumbered by a ballot
// prefix count.
__device__ inline double readlane_f64(double v, int j) {
    const long long u = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane(static_cast<int>(u & 0xffffffffll), j);
    const int hi = __builtin_amdgcn_readlane(static_cast<int>(u >> 32), j);
    return __longlong_as_double((static_cast<long long>(hi) << 32) |
                                static_cast<long long>(static_cast<unsigned>(lo)));
}

__global__ __launch_bounds__(64) void tree_prune_wave_kernel(
    const int32_t* __restrict__ parent, const float* __restrict__ logq, int M, double tau,
    int budget, double* __restrict__ cum, int32_t* __restrict__ new_index,
    int32_t* __restrict__ new_parent, int32_t* __restrict__ count) {
    __shared__ int old_of_new[64];
    const int b = blockIdx.x, i = threadIdx.x;
    const bool node = i < M;
    const size_t base = static_cast<size_t>(b) * M;
    const int p = node ? parent[base + i] : -1;
    const float lq = node ? logq[base + i] : 0.0f;
    const bool bad = node && (i == 0 ? p != -1 : (p < 0 || p >= i || !(lq <= 0.0f)));
    if (__ballot(bad)) {
        if (node) {
            cum[base + i] = __builtin_nan("");
            new_index[base + i] = -1;
            new_parent[base + i] = -1;
        }
        if (i == 0)
            count[b] = -1;
        return;
    }
    // Every parent now lies in [0, i) (the root's is -1): one level per round.
    const int src = p >= 0 ? p : 0;
    double c = 0.0;
    bool ready = i == 0 || !node;
    while (__ballot(!ready)) {
        const double cp = __shfl(c, src, 64);
        const int rp = __shfl(ready ? 1 : 0, src, 64);
        if (!ready && rp) {
            c = cp + static_cast<double>(lq);
            ready = true;
        }
    }
    int rank = 0;
    for (int j = 0; j < M; ++j) {
        const double cj = readlane_f64(c, j);
        rank += (cj > c || (cj == c && j < i)) ? 1 : 0;
    }
    const bool keep = node && c >= tau && rank < budget;
    const unsigned long long m = __ballot(keep);
    const int before = __builtin_amdgcn_mbcnt_hi(static_cast<unsigned>(m >> 32),
                                                 __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(m), 0));
    const int total = __popcll(m);
    const int ni = keep ? before : -1;
    if (keep)
        old_of_new[before] = i;
    __syncthreads();
    // New node i < total is old node `old`; its new parent is the new index
    // of old's parent (-1 for the root).
    const int old = i < total ? old_of_new[i] : 0;
    const int p_old = __shfl(p, old, 64);
    const int ni_of_p = __shfl(ni, p_old >= 0 ? p_old : 0, 64);
    if (node) {
        cum[base + i] = c;
        new_index[base + i] = ni;
        new_parent[base + i] = i < total && old != 0 ? ni_of_p : -1;
    }
    if (i == 0)
        count[b] = total;
}

struct ArgPart {
    float v;
    int idx;
};

// Raw-logit argmax of one split of one node's target row; lowest index wins
// a tie (each thread walks its groups in index order, merges compare keys).
template <int DT, bool VEC>
__global__ __launch_bounds__(kBlock) void tree_argmax_kernel(
    const void* __restrict__ target, const int32_t* __restrict__ n_nodes, int M, int vocab,
    int nsplit, ArgPart* __restrict__ part) {
    using Ld = Loader<DT, VEC>;
    constexpr int W = Ld::W;
    __shared__ float sv[kWaves];
    __shared__ int si[kWaves];
    const long row = blockIdx.x;
    const int b = static_cast<int>(row / M), x = static_cast<int>(row % M);
    const int n = n_nodes[b];
    if (n < 1 || n > M || x >= n)
        return;  // rows the walk never reads
    const int c = blockIdx.y;
    const long groups = vocab / W;
    long g0, g1;
    split_range(groups, nsplit, c, &g0, &g1);
    const void* rp = row_ptr(target, DT, static_cast<size_t>(row), vocab);
    float bv = -__builtin_huge_valf();
    int bi = 0x7fffffff;
    for (long g = g0 + threadIdx.x; g < g1; g += kBlock) {
        float z[W];
        Ld::unpack(Ld::load_nt(rp, g), z);
#pragma unroll
        for (int e = 0; e < W; ++e)
            if (z[e] > bv) {
                bv = z[e];
                bi = static_cast<int>(g * W + e);
            }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (ov > bv || (ov == bv && oi < bi)) {
            bv = ov;
            bi = oi;
        }
    }
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) {
        sv[w] = bv;
        si[w] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int v = 1; v < kWaves; ++v)
            if (sv[v] > bv || (sv[v] == bv && si[v] < bi)) {
                bv = sv[v];
                bi = si[v];
            }
        part[row * nsplit + c] = ArgPart{bv, bi};
    }
}

__global__ __launch_bounds__(64) void tree_walk_kernel(
    const int32_t* __restrict__ parent, const int32_t* __restrict__ token,
    const int32_t* __restrict__ n_nodes, int M, int vocab, int nsplit,
    const ArgPart* __restrict__ part, int32_t* __restrict__ out_len, int32_t* __restrict__ out_path,
    int32_t* __restrict__ out_extra) {
    __shared__ int path[SPEC_TREE_MAX_NODES];
    const int b = blockIdx.x, lane = threadIdx.x;
    const size_t base = static_cast<size_t>(b) * M;
    const int n = n_nodes[b];
    bool bad = n < 1 || n > M;
    if (!bad) {
        for (int j = lane; j < n; j += 64) {
            const int p = parent[base + j];
            if (j == 0 ? p != -1 : (p < 0 || p >= j || token[base + j] < 0 || token[base + j] >= vocab))
                bad = true;
        }
    }
    bad = __ballot(bad) != 0ull;
    int L = 0, extra = -1;
    if (!bad) {
        int x = 0;
        for (;;) {
            // argmax of row x: merge its splits
            float bv = -__builtin_huge_valf();
            int bi = 0x7fffffff;
            for (int c = lane; c < nsplit; c += 64) {
                const ArgPart q = part[(base + x) * nsplit + c];
                if (q.v > bv || (q.v == bv && q.idx < bi)) {
                    bv = q.v;
                    bi = q.idx;
                }
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                const float ov = __shfl_xor(bv, o, 64);
                const int oi = __shfl_xor(bi, o, 64);
                if (ov > bv || (ov == bv && oi < bi)) {
                    bv = ov;
                    bi = oi;
                }
            }
            if (!(bv > -__builtin_huge_valf())) {
                bad = true;  // a reached row with no finite logit
                break;
            }
            int next = -1;
            for (int j0 = 1; j0 < n && next < 0; j0 += 64) {
                const int j = j0 + lane;
                const bool match = j < n && parent[base + j] == x && token[base + j] == bi;
                const unsigned long long m = __ballot(match);
                if (m)
                    next = j0 + __ffsll(static_cast<long long>(m)) - 1;
            }
            if (next < 0) {
                extra = bi;
                break;
            }
            if (lane == 0)
                path[L] = next;
            ++L;
            x = next;
        }
    }
    __syncthreads();
    for (int j = lane; j < M; j += 64)
        out_path[base + j] = (!bad && j < L) ? path[j] : -1;
    if (lane == 0) {
        out_len[b] = bad ? -1 : L;
        out_extra[b] = bad ? -1 : extra;
    }
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace
}  // namespace specv

using namespace specv;

struct spec_tree_ctx {
    int B = 0, M = 0, V = 0, dtype = 0, nsplit = 1;
    hipStream_t stream = nullptr;
    ArgPart* part = nullptr;
    // Sampled verification: trees in flight at once, the parts' exchange
    // slots followed by the kernel's three control words, and the polls a
    // part makes before giving up on a partner.
    int sample_groups = 0;
    uint64_t* shares = nullptr;
    uint64_t* ctl = nullptr;
    int spin_limit = 0;
};

extern "C" {

int spec_tree_prune(int batch, int nodes, const int32_t* parent, const float* logq, double tau,
                    int budget, double* out_cum, int32_t* out_new_index,
                    int32_t* out_new_parent, int32_t* out_count, void* hip_stream) {
    if (batch < 0 || nodes < 1 || nodes > SPEC_TREE_MAX_NODES || budget < 1 || !(tau <= 0.0))
        return SPEC_EINVAL;
    if (batch == 0)
        return SPEC_OK;
    if (!parent || !logq || !out_cum || !out_new_index || !out_new_parent || !out_count ||
        !aligned(parent, 4) || !aligned(logq, 4) || !aligned(out_cum, 8) ||
        !aligned(out_new_index, 4) || !aligned(out_new_parent, 4) || !aligned(out_count, 4))
        return SPEC_EINVAL;
    if (nodes <= 64)
        tree_prune_wave_kernel<<<dim3(static_cast<unsigned>(batch)), dim3(64), 0,
                                 static_cast<hipStream_t>(hip_stream)>>>(
            parent, logq, nodes, tau, budget, out_cum, out_new_index, out_new_parent, out_count);
    else
        tree_prune_kernel<<<dim3(static_cast<unsigned>(batch)), dim3(kTreeThreads), 0,
                            static_cast<hipStream_t>(hip_stream)>>>(parent, logq, nodes, tau,
                                                                    budget, out_cum, out_new_index,
                                                                    out_new_parent, out_count);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

int spec_tree_verify_init(int batch, int max_nodes, int vocab, int dtype, void* hip_stream,
                          spec_tree_ctx** out_ctx) {
    if (!out_ctx)
        return SPEC_EINVAL;
    *out_ctx = nullptr;
    if (batch < 1 || max_nodes < 1 || max_nodes > SPEC_TREE_MAX_NODES || vocab < 1 ||
        (dtype != SPEC_F32 && dtype != SPEC_BF16))
        return SPEC_EINVAL;
    const long rows = static_cast<long>(batch) * max_nodes;
    if (rows >= (1L << 31))
        return SPEC_EINVAL;
    spec_tree_ctx* ctx = new (std::nothrow) spec_tree_ctx();
    if (!ctx)
        return SPEC_ENOMEM;
    ctx->B = batch;
    ctx->M = max_nodes;
    ctx->V = vocab;
    ctx->dtype = dtype;
    ctx->stream = static_cast<hipStream_t>(hip_stream);
    // About 8192 workgroups, at least 1024 16-byte groups each, at most 64 splits.
    const long groups = vocab / (dtype == SPEC_BF16 ? 8 : 4);
    long n = (8192 + rows - 1) / rows;
    n = std::min(n, std::max(1L, groups / 1024));
    ctx->nsplit = static_cast<int>(std::max(1L, std::min(n, 64L)));
    if (hipMalloc(&ctx->part, static_cast<size_t>(rows) * ctx->nsplit * sizeof(ArgPart)) != hipSuccess) {
        delete ctx;
        return SPEC_ENOMEM;
    }
    int sample_groups = 0;
    if (tree_sample_max_groups(dtype, &sample_groups) != hipSuccess || sample_groups < 1) {
        (void)hipFree(ctx->part);
        delete ctx;
        return SPEC_EHIP;
    }
    ctx->sample_groups = std::min(sample_groups, batch);
    const size_t share_bytes = static_cast<size_t>(ctx->sample_groups) * tree_sample_group_bytes();
    const size_t ctl_words = 4;
    ctx->spin_limit = tree_sample_default_spin_limit();
    if (hipMalloc(reinterpret_cast<void**>(&ctx->shares), share_bytes + ctl_words * 8) != hipSuccess ||
        hipMemset(ctx->shares, 0, share_bytes + ctl_words * 8) != hipSuccess) {
        (void)hipFree(ctx->shares);
        (void)hipFree(ctx->part);
        delete ctx;
        return SPEC_ENOMEM;
    }
    ctx->ctl = ctx->shares + share_bytes / 8;
    *out_ctx = ctx;
    return SPEC_OK;
}

int spec_tree_verify_set_spin_limit(spec_tree_ctx* ctx, int polls) {
    if (!ctx || polls < 0)
        return SPEC_EINVAL;
    ctx->spin_limit = polls;
    return SPEC_OK;
}

int spec_tree_verify_gave_up(spec_tree_ctx* ctx, uint64_t* out_count) {
    if (!ctx || !out_count)
        return SPEC_EINVAL;
    if (hipStreamSynchronize(ctx->stream) != hipSuccess ||
        hipMemcpy(out_count, ctx->ctl + 2, sizeof(uint64_t), hipMemcpyDeviceToHost) != hipSuccess)
        return SPEC_EHIP;
    return SPEC_OK;
}

int spec_tree_verify_set_stream(spec_tree_ctx* ctx, void* hip_stream) {
    if (!ctx)
        return SPEC_EINVAL;
    ctx->stream = static_cast<hipStream_t>(hip_stream);
    return SPEC_OK;
}

int spec_tree_verify_greedy(spec_tree_ctx* ctx, const int32_t* parent, const int32_t* token,
                            const int32_t* n_nodes, const void* target, int32_t* out_length,
                            int32_t* out_path, int32_t* out_extra) {
    if (!ctx || !parent || !token || !n_nodes || !target || !out_length || !out_path || !out_extra)
        return SPEC_EINVAL;
    const size_t esz = ctx->dtype == SPEC_BF16 ? 2 : 4;
    if (!aligned(parent, 4) || !aligned(token, 4) || !aligned(n_nodes, 4) || !aligned(target, esz) ||
        !aligned(out_length, 4) || !aligned(out_path, 4) || !aligned(out_extra, 4))
        return SPEC_EINVAL;
    const int W = ctx->dtype == SPEC_BF16 ? 8 : 4;
    const bool vec = ctx->V % W == 0 && aligned(target, 16);
    const dim3 grid(static_cast<unsigned>(static_cast<long>(ctx->B) * ctx->M),
                    static_cast<unsigned>(ctx->nsplit));
    hipStream_t s = ctx->stream;
    if (ctx->dtype == SPEC_BF16) {
        if (vec)
            tree_argmax_kernel<kBF16, true><<<grid, dim3(kBlock), 0, s>>>(target, n_nodes, ctx->M, ctx->V, ctx->nsplit, ctx->part);
        else
            tree_argmax_kernel<kBF16, false><<<grid, dim3(kBlock), 0, s>>>(target, n_nodes, ctx->M, ctx->V, ctx->nsplit, ctx->part);
    } else {
        if (vec)
            tree_argmax_kernel<kF32, true><<<grid, dim3(kBlock), 0, s>>>(target, n_nodes, ctx->M, ctx->V, ctx->nsplit, ctx->part);
        else
            tree_argmax_kernel<kF32, false><<<grid, dim3(kBlock), 0, s>>>(target, n_nodes, ctx->M, ctx->V, ctx->nsplit, ctx->part);
    }
    if (hipGetLastError() != hipSuccess)
        return SPEC_EHIP;
    tree_walk_kernel<<<dim3(static_cast<unsigned>(ctx->B)), dim3(64), 0, s>>>(
        parent, token, n_nodes, ctx->M, ctx->V, ctx->nsplit, ctx->part, out_length, out_path,
        out_extra);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

int spec_tree_verify_sample(spec_tree_ctx* ctx, const int32_t* parent, const int32_t* token,
                            const int32_t* n_nodes, const void* draft, const void* target,
                            const float* temperature, uint64_t seed, uint64_t offset,
                            int32_t* out_length, int32_t* out_path, int32_t* out_extra) {
    if (!ctx || !parent || !token || !n_nodes || !draft || !target || !temperature ||
        !out_length || !out_path || !out_extra)
        return SPEC_EINVAL;
    const size_t esz = ctx->dtype == SPEC_BF16 ? 2 : 4;
    if (!aligned(parent, 4) || !aligned(token, 4) || !aligned(n_nodes, 4) || !aligned(draft, esz) ||
        !aligned(target, esz) || !aligned(temperature, 4) || !aligned(out_length, 4) ||
        !aligned(out_path, 4) || !aligned(out_extra, 4))
        return SPEC_EINVAL;
    if (!tree_sample_fits(ctx->V, ctx->dtype))
        return SPEC_EINVAL;
    // Exchange tags carry 20 bits of pass count per launch.
    const long trees_per_group = (ctx->B + ctx->sample_groups - 1) / ctx->sample_groups;
    if (trees_per_group * (2L * ctx->M + 2) >= (1L << 20))
        return SPEC_EINVAL;
    const int W = ctx->dtype == SPEC_BF16 ? 8 : 4;
    const bool vec = ctx->V % W == 0 && aligned(draft, 16) && aligned(target, 16);
    const hipError_t e = launch_tree_sample(ctx->B, ctx->M, ctx->V, ctx->dtype, vec, parent, token,
                                            n_nodes, draft, target, temperature, seed, offset,
                                            out_length, out_path, out_extra, ctx->shares,
                                            ctx->ctl, ctx->spin_limit, ctx->sample_groups,
                                            ctx->stream);
    return e == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

int spec_tree_verify_destroy(spec_tree_ctx* ctx) {
    if (!ctx)
        return SPEC_EINVAL;
    int rc = SPEC_OK;
    if (hipStreamSynchronize(ctx->stream) != hipSuccess)
        rc = SPEC_EHIP;
    if (ctx->part && hipFree(ctx->part) != hipSuccess)
        rc = SPEC_EHIP;
    if (ctx->shares && hipFree(ctx->shares) != hipSuccess)
        rc = SPEC_EHIP;
    delete ctx;
    return rc;
}

}  // extern "C"
