// Low-rank draft LM head z = W_up W_down h with its fused row normaliser
// (SlimSpec summary, Methodology, architecture: the full V x d head is
// factored through rank r, computed with dense matrix products).
//
// Both products run on the matrix cores (v_mfma_f32_16x16x32_bf16: bf16
// operands, binary32 accumulation). One tile routine serves both: C[m][n] =
// sum_k A[m][k] B[n][k] with A and B row-major and K contiguous, a 128 x 128
// output tile per 256-thread workgroup (2 x 2 wavefronts of 64 x 64, i.e. 4 x 4
// MFMA tiles each), K in chunks of 64 staged through LDS with double
// buffering (rows padded to 144 bytes) and two chunks in flight in registers.
//
//   head_down: u = W_down h, split over K into fp32 partials (the activation
//     is small, N x r, so the split gives the GPU enough workgroups);
//   head_down_reduce: u = bf16(sum of the partials, in split order);
//   head_up: z = W_up u; the tile is rounded to bf16, staged in LDS, stored
//     with 16-byte rows, and, while it is still on chip, reduced to one
//     (m, s) pair per row: m = fl32(max x * log2e), s = sum 2^(fma(x, log2e,
//     -m)) with x = fl32(z * fl32(1/T)), the row kernel's base-2 form;
//   head_lse: merges a row's (m, s) pairs into its log-normaliser.
// Workgroups of head_up are ordered row tile fastest, so the workgroups that
// read one W_up tile run together and all but the first read it from cache.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <new>

#include "spec_head.h"

namespace specv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLdsK = kBK + 8;    // bf16 per LDS row of a K chunk (144 bytes)
constexpr int kThreads = 256;
constexpr int kOutLd = kBN + 8;   // bf16 per LDS row of the staged output tile
constexpr int kLdsElems = 2 * (kBM + kBN) * kLdsK;
constexpr float kHeadLog2e = 1.44269504088896340736f;

static_assert(kBM * kOutLd <= kLdsElems, "output staging must fit the K-chunk buffers");

struct HeadPart {
    float m;
    int pad;
    double s;
};

__device__ inline uint16_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }

// Temperature classification of the verifier: returns false unless T > 0,
// finite, with a finite correctly rounded reciprocal.
__device__ inline bool sampled_row(float t, float* inv_t) {
    if (!(t > 0.0f) || t == __builtin_huge_valf())
        return false;
    const float r = 1.0f / t;
    if (r == __builtin_huge_valf())
        return false;
    *inv_t = r;
    return true;
}

struct TileArgs {
    const uint16_t* A;  // [M][K]
    const uint16_t* B;  // [Nc][K]
    int M, Nc, K;
    int m0, n0;
};

// A row past the end reads row 0 instead: its products land only in output
// rows or columns that are never stored. With no branch and no select on the
// loaded value, the compiler waits for exactly the loads it needs.
__device__ inline u32x4 load16(const uint16_t* base, long row, int ld, int k, bool ok) {
    return *reinterpret_cast<const u32x4*>(base + (ok ? row : 0L) * ld + k);
}

// acc[mt][nt] += the wavefront's 64 x 64 block of A[m0.., k] B[n0.., k]^T over
// k in [k_begin, k_end) (a multiple of 64). Lane l of MFMA tile (mt, nt) ends
// up holding C[row][col] for row = wm*64 + mt*16 + 4*(l/16) + j, j < 4, and
// col = wn*64 + nt*16 + l%16. Rows or columns past M or Nc hold garbage
// (finite: products of real rows) that the callers never store.
// Pipeline: chunk c is multiplied out of LDS buffer c % 2 while chunks c + 1
// and c + 2 are in registers; after the multiply, chunk c + 1 goes to the
// other LDS buffer and its registers start loading chunk c + 3.
struct ChunkRegs {
    u32x4 a[4], b[4];
};

__device__ inline void tile_mma(const TileArgs& t, int k_begin, int k_end, uint16_t* lds,
                                f32x4 (&acc)[4][4]) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    uint16_t* la = lds;
    uint16_t* lb = lds + 2 * kBM * kLdsK;
    const int nk = (k_end - k_begin) / kBK;
    // Chunks past the end reload the last one (never stored where it is read).
    auto gload = [&](ChunkRegs& R, int c) {
        const int k0 = k_begin + (c < nk ? c : nk - 1) * kBK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + kThreads * i;       // 1024 16-byte pieces per operand
            const int row = q >> 3, kc = (q & 7) * 8;
            R.a[i] = load16(t.A, t.m0 + row, t.K, k0 + kc, t.m0 + row < t.M);
            R.b[i] = load16(t.B, t.n0 + row, t.K, k0 + kc, t.n0 + row < t.Nc);
        }
    };
    auto lstore = [&](const ChunkRegs& R, int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + kThreads * i;
            const int row = q >> 3, kc = (q & 7) * 8;
            *reinterpret_cast<u32x4*>(la + (buf * kBM + row) * kLdsK + kc) = R.a[i];
            *reinterpret_cast<u32x4*>(lb + (buf * kBN + row) * kLdsK + kc) = R.b[i];
        }
    };
    const int fr = lane & 15, fk = (lane >> 4) * 8;
    auto multiply = [&](int buf) {
#pragma unroll
        for (int ks = 0; ks < kBK; ks += 32) {
            bf16x8 a[4], b[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                a[mt] = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(
                                la + (buf * kBM + wm * 64 + mt * 16 + fr) * kLdsK + ks + fk));
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
                b[nt] = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(
                                lb + (buf * kBN + wn * 64 + nt * 16 + fr) * kLdsK + ks + fk));
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
                    acc[mt][nt] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt], b[nt], acc[mt][nt], 0, 0, 0);
        }
    };
    if (nk <= 0)
        return;
    ChunkRegs r0, r1;
    gload(r0, 0);
    lstore(r0, 0);
    gload(r0, 1);
    gload(r1, 2);
    __syncthreads();
    // Two iterations per trip so that the register sets have fixed names. The
    // stores and loads past the last chunk are unconditional too: they fill an
    // LDS buffer that is not read again.
    for (int c = 0; c < nk; c += 2) {
        multiply(0);
        lstore(r0, 1);
        gload(r0, c + 3);
        __syncthreads();
        if (c + 1 >= nk)
            break;
        multiply(1);
        lstore(r1, 0);
        gload(r1, c + 4);
        __syncthreads();
    }
}

__device__ inline void zero(f32x4 (&acc)[4][4]) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
            acc[mt][nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

// partial[z][n][j] = sum over split z's K range of h[n][k] w_down[j][k].
__global__ __launch_bounds__(kThreads) void head_down_kernel(const uint16_t* __restrict__ h,
                                                             const uint16_t* __restrict__ w_down,
                                                             int N, int r, int d, int k_per_split,
                                                             float* __restrict__ partial) {
    __shared__ __align__(16) uint16_t lds[kLdsElems];
    const TileArgs t{h, w_down, N, r, d, static_cast<int>(blockIdx.x) * kBM,
                     static_cast<int>(blockIdx.y) * kBN};
    const int kb = static_cast<int>(blockIdx.z) * k_per_split;
    const int ke = kb + k_per_split < d ? kb + k_per_split : d;
    f32x4 acc[4][4];
    zero(acc);
    tile_mma(t, kb, ke, lds, acc);
    float* out = partial + static_cast<size_t>(blockIdx.z) * N * r;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w >> 1, wn = w & 1;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = t.m0 + wm * 64 + mt * 16 + 4 * (lane >> 4) + j;
                const int col = t.n0 + wn * 64 + nt * 16 + (lane & 15);
                if (row < N && col < r)
                    out[static_cast<size_t>(row) * r + col] = acc[mt][nt][j];
            }
}

// n is a multiple of 32 (r is), so every thread takes four consecutive values.
__global__ __launch_bounds__(256) void head_down_reduce_kernel(const float* __restrict__ partial,
                                                               int splits, long n,
                                                               uint16_t* __restrict__ u) {
    const long n4 = n / 4;
    for (long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n4;
         i += static_cast<long>(gridDim.x) * blockDim.x) {
        float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        for (int z = 0; z < splits; ++z) {
            const float4 v = reinterpret_cast<const float4*>(partial + static_cast<size_t>(z) * n)[i];
            s.x += v.x;
            s.y += v.y;
            s.z += v.z;
            s.w += v.w;
        }
        const uint32_t lo = bf16_rne(s.x) | (static_cast<uint32_t>(bf16_rne(s.y)) << 16);
        const uint32_t hi = bf16_rne(s.z) | (static_cast<uint32_t>(bf16_rne(s.w)) << 16);
        reinterpret_cast<uint2*>(u)[i] = make_uint2(lo, hi);
    }
}

// z = bf16(u w_up^T) for one 128-row x 128-vocabulary tile, and each row's
// (m, s) over the tile's columns.
__global__ __launch_bounds__(kThreads) void head_up_kernel(const uint16_t* __restrict__ u,
                                                           const uint16_t* __restrict__ w_up,
                                                           const float* __restrict__ temperature,
                                                           int N, int V, int r,
                                                           uint16_t* __restrict__ z,
                                                           HeadPart* __restrict__ part, int ntn) {
    __shared__ __align__(16) uint16_t lds[kLdsElems];
    const TileArgs t{u, w_up, N, V, r, static_cast<int>(blockIdx.x) * kBM,
                     static_cast<int>(blockIdx.y) * kBN};
    f32x4 acc[4][4];
    zero(acc);
    tile_mma(t, 0, r, lds, acc);  // ends with a barrier: the LDS is free

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    uint16_t* st = lds;  // [kBM][kOutLd]
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = wm * 64 + mt * 16 + 4 * (lane >> 4) + j;
                const int col = wn * 64 + nt * 16 + (lane & 15);
                st[row * kOutLd + col] = bf16_rne(acc[mt][nt][j]);
            }
    __syncthreads();

    // 16-byte stores: a row of the tile is 16 chunks of 8 logits.
#pragma unroll
    for (int i = 0; i < (kBM * kBN / 8) / kThreads; ++i) {
        const int c = tid + kThreads * i;
        const int row = c >> 4, cc = (c & 15) * 8;
        if (t.m0 + row < N && t.n0 + cc < V)
            *reinterpret_cast<u32x4*>(z + static_cast<size_t>(t.m0 + row) * V + t.n0 + cc) =
                *reinterpret_cast<const u32x4*>(st + row * kOutLd + cc);
    }

    // Row normaliser pieces: two threads per row, 64 columns each.
    const int row = tid >> 1, half = tid & 1;
    const int grow = t.m0 + row;
    const int n_valid = V - t.n0 < kBN ? V - t.n0 : kBN;
    float inv_t = 0.0f;
    const bool active = grow < N && sampled_row(temperature[grow < N ? grow : 0], &inv_t);
    const int c0 = half * 64;
    const int c1 = c0 + 64 < n_valid ? c0 + 64 : n_valid;
    float xmax = -__builtin_huge_valf();
    if (active)
        for (int c = c0; c < c1; ++c)
            xmax = fmaxf(xmax, bf16_to_f32(st[row * kOutLd + c]) * inv_t);
    xmax = fmaxf(xmax, __shfl_xor(xmax, 1, 64));
    const float m = xmax * kHeadLog2e;
    double s = 0.0;
    if (active && xmax > -__builtin_huge_valf()) {
        for (int c = c0; c < c1; c += 8) {
            float g = 0.0f;  // eight terms in binary32, then binary64
            const int ce = c + 8 < c1 ? c + 8 : c1;
            for (int e = c; e < ce; ++e) {
                const float x = bf16_to_f32(st[row * kOutLd + e]) * inv_t;
                g += __builtin_amdgcn_exp2f(__builtin_fmaf(x, kHeadLog2e, -m));
            }
            s += static_cast<double>(g);
        }
    }
    s += __shfl_xor(s, 1, 64);
    if (half == 0 && grow < N)
        part[static_cast<size_t>(grow) * ntn + blockIdx.y] = HeadPart{m, 0, s};
}

// One 256-thread workgroup per row: each thread folds a few (m, s) pieces,
// then the wavefronts and the workgroup combine them in a fixed order.
__global__ __launch_bounds__(256) void head_lse_kernel(const HeadPart* __restrict__ part, int ntn,
                                                       const float* __restrict__ temperature,
                                                       double* __restrict__ lse) {
    __shared__ float lm[4];
    __shared__ double ls[4];
    const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    float inv_t;
    if (!sampled_row(temperature[row], &inv_t)) {
        if (tid == 0)
            lse[row] = __builtin_nan("");
        return;
    }
    const HeadPart* p = part + static_cast<size_t>(row) * ntn;
    float M = -__builtin_huge_valf();
    for (int c = tid; c < ntn; c += 256)
        M = fmaxf(M, p[c].m);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        M = fmaxf(M, __shfl_xor(M, o, 64));
    if (lane == 0)
        lm[w] = M;
    __syncthreads();
    M = fmaxf(fmaxf(lm[0], lm[1]), fmaxf(lm[2], lm[3]));
    double S = 0.0;
    for (int c = tid; c < ntn; c += 256) {
        const HeadPart q = p[c];
        if (q.s > 0.0) {
            // exactly 1 for the pieces holding the maximum; a binary32 factor otherwise
            const float f = q.m == M ? 1.0f : __builtin_amdgcn_exp2f(q.m - M);
            S += q.s * static_cast<double>(f);
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        S += __shfl_xor(S, o, 64);
    if (lane == 0)
        ls[w] = S;
    __syncthreads();
    if (tid == 0) {
        const double tot = (ls[0] + ls[1]) + (ls[2] + ls[3]);
        lse[row] = (static_cast<double>(M) + log2(tot)) / static_cast<double>(kHeadLog2e);
    }
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace
}  // namespace specv

using namespace specv;

struct spec_head_ctx {
    int N = 0, d = 0, r = 0, V = 0;
    int splits = 1, k_per_split = 0, ntn = 0;
    hipStream_t stream = nullptr;
    void* ws = nullptr;
    uint16_t* u = nullptr;
    float* partial = nullptr;
    HeadPart* part = nullptr;
};

extern "C" {

int spec_lowrank_head_init(int rows, int hidden, int rank, int vocab, void* hip_stream,
                           spec_head_ctx** out_ctx) {
    if (!out_ctx)
        return SPEC_EINVAL;
    *out_ctx = nullptr;
    if (rows < 1 || hidden < kBK || hidden % kBK || rank < kBK || rank % kBK || vocab < 8 ||
        vocab % 8 || (vocab + kBN - 1) / kBN > 65535)
        return SPEC_EINVAL;
    spec_head_ctx* ctx = new (std::nothrow) spec_head_ctx();
    if (!ctx)
        return SPEC_ENOMEM;
    ctx->N = rows;
    ctx->d = hidden;
    ctx->r = rank;
    ctx->V = vocab;
    ctx->stream = static_cast<hipStream_t>(hip_stream);
    // Split the small first product over K until there are ~128 workgroups,
    // keeping at least 4 chunks per split.
    const int tiles = ((rows + kBM - 1) / kBM) * ((rank + kBN - 1) / kBN);
    const int max_split = std::max(1, hidden / (4 * kBK));
    ctx->splits = std::max(1, std::min(max_split, (128 + tiles - 1) / tiles));
    const int chunks = hidden / kBK;
    ctx->k_per_split = ((chunks + ctx->splits - 1) / ctx->splits) * kBK;
    ctx->splits = (hidden + ctx->k_per_split - 1) / ctx->k_per_split;
    ctx->ntn = (vocab + kBN - 1) / kBN;
    const size_t nr = static_cast<size_t>(rows) * rank;
    size_t off = 0;
    const size_t o_u = off;
    off = align_up(off + nr * sizeof(uint16_t), 256);
    const size_t o_p = off;
    off = align_up(off + nr * ctx->splits * sizeof(float), 256);
    const size_t o_h = off;
    off = align_up(off + static_cast<size_t>(rows) * ctx->ntn * sizeof(HeadPart), 256);
    if (hipMalloc(&ctx->ws, off) != hipSuccess) {
        delete ctx;
        return SPEC_ENOMEM;
    }
    char* base = static_cast<char*>(ctx->ws);
    ctx->u = reinterpret_cast<uint16_t*>(base + o_u);
    ctx->partial = reinterpret_cast<float*>(base + o_p);
    ctx->part = reinterpret_cast<HeadPart*>(base + o_h);
    *out_ctx = ctx;
    return SPEC_OK;
}

int spec_lowrank_head_set_stream(spec_head_ctx* ctx, void* hip_stream) {
    if (!ctx)
        return SPEC_EINVAL;
    ctx->stream = static_cast<hipStream_t>(hip_stream);
    return SPEC_OK;
}

int spec_lowrank_head(spec_head_ctx* ctx, const void* hidden, const void* w_down,
                      const void* w_up, const float* temperature, void* out_logits,
                      double* out_lse) {
    if (!ctx || !hidden || !w_down || !w_up || !temperature || !out_logits || !out_lse)
        return SPEC_EINVAL;
    if (!aligned(hidden, 16) || !aligned(w_down, 16) || !aligned(w_up, 16) ||
        !aligned(out_logits, 16) || !aligned(temperature, 4) || !aligned(out_lse, 8))
        return SPEC_EINVAL;
    const int N = ctx->N, d = ctx->d, r = ctx->r, V = ctx->V;
    hipStream_t s = ctx->stream;
    const unsigned mt = static_cast<unsigned>((N + kBM - 1) / kBM);
    head_down_kernel<<<dim3(mt, static_cast<unsigned>((r + kBN - 1) / kBN),
                            static_cast<unsigned>(ctx->splits)),
                       dim3(kThreads), 0, s>>>(static_cast<const uint16_t*>(hidden),
                                              static_cast<const uint16_t*>(w_down), N, r, d,
                                              ctx->k_per_split, ctx->partial);
    if (hipGetLastError() != hipSuccess)
        return SPEC_EHIP;
    const long nr = static_cast<long>(N) * r;
    const unsigned rb = static_cast<unsigned>(std::min<long>((nr / 4 + 255) / 256, 4096));
    head_down_reduce_kernel<<<dim3(rb), dim3(256), 0, s>>>(ctx->partial, ctx->splits, nr, ctx->u);
    if (hipGetLastError() != hipSuccess)
        return SPEC_EHIP;
    head_up_kernel<<<dim3(mt, static_cast<unsigned>(ctx->ntn)), dim3(kThreads), 0, s>>>(
        ctx->u, static_cast<const uint16_t*>(w_up), temperature, N, V, r,
        static_cast<uint16_t*>(out_logits), ctx->part, ctx->ntn);
    if (hipGetLastError() != hipSuccess)
        return SPEC_EHIP;
    head_lse_kernel<<<dim3(static_cast<unsigned>(N)), dim3(256), 0, s>>>(ctx->part, ctx->ntn,
                                                                         temperature, out_lse);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

int spec_lowrank_head_copy_activation(spec_head_ctx* ctx, void* out_u) {
    if (!ctx || !out_u)
        return SPEC_EINVAL;
    const size_t bytes = static_cast<size_t>(ctx->N) * ctx->r * sizeof(uint16_t);
    return hipMemcpyAsync(out_u, ctx->u, bytes, hipMemcpyDeviceToDevice, ctx->stream) == hipSuccess
               ? SPEC_OK
               : SPEC_EHIP;
}

int spec_lowrank_head_destroy(spec_head_ctx* ctx) {
    if (!ctx)
        return SPEC_EINVAL;
    int rc = SPEC_OK;
    if (hipStreamSynchronize(ctx->stream) != hipSuccess)
        rc = SPEC_EHIP;
    if (ctx->ws && hipFree(ctx->ws) != hipSuccess)
        rc = SPEC_EHIP;
    delete ctx;
    return rc;
}

}  // extern "C"
