// Low-rank draft LM head z = W_up W_down h with its fused row normaliser
// (SlimSpec summary, Methodology, architecture: the full V x d head is
// factored through rank r, computed with dense matrix products).
//
// Both products run on the matrix cores (v_mfma_f32_16x16x32_bf16: bf16
// operands, binary32 accumulation).
//
//   head_down: u = bf16(W_down h), one workgroup per 16 x 32 tile of u whose
//     16 wavefronts split K and add their binary32 partial tiles in LDS;
//   head_up_stream (rank 256 or 512): z^T = W_up u^T with the vocabulary on
//     M, one workgroup per CU streaming its run of W_up through an LDS ring
//     while the batch rows stay in registers; each block of logits is rounded
//     to bf16, stored, and folded into per-row (m, s) pairs while still in
//     registers: m = fl32(max x * log2e), s = sum 2^(fma(x, log2e, -m)) with
//     x = fl32(z * fl32(1/T)), the row kernel's base-2 form;
//   head_up (other ranks): the same product with the tile routine below
//     (C[m][n] = sum_k A[m][k] B[n][k], A and B row-major with K contiguous,
//     64 x 64 per wavefront, K in chunks of 64 staged through LDS with double
//     buffering, rows padded to 144 bytes, and two chunks in flight in
//     registers), 128 vocabulary entries x 256 batch rows per workgroup;
//   head_lse: merges a row's (m, s) pairs into its log-normaliser.
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
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBK = 64;
constexpr int kLdsK = kBK + 8;    // bf16 per LDS row of a K chunk (144 bytes)
constexpr float kHeadLog2e = 1.44269504088896340736f;

// Tile shape of the second product with the tile routine: the vocabulary on
// M and all of a 256-row batch on N, so each W_up slab is read once and every
// lane ends up holding four consecutive logits of one row.
constexpr int kUpBM = 128, kUpBN = 256;       // 2 x 4 wavefronts of 64 x 64
constexpr int kUpThreads = 512;

template <int BM, int BN>
constexpr int lds_elems() { return 2 * (BM + BN) * kLdsK; }

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
// k in [k_begin, k_end) (a multiple of 64); the THREADS / 64 wavefronts form a
// (BM / 64) x (BN / 64) grid, wavefront w at (wm, wn) = (w / (BN/64), w % (BN/64)).
// Lane l of MFMA tile (mt, nt) ends up holding C[row][col] for
// row = wm*64 + mt*16 + 4*(l/16) + j, j < 4, and col = wn*64 + nt*16 + l%16.
// Rows or columns past M or Nc hold garbage (finite: products of real rows)
// that the callers never store.
// Pipeline: chunk c is multiplied out of LDS buffer c % 2 while chunks c + 1
// and c + 2 are in registers; after the multiply, chunk c + 1 goes to the
// other LDS buffer and its registers start loading chunk c + 3.
template <int BM, int BN, int THREADS>
struct ChunkRegs {
    static constexpr int kA = BM * (kBK / 8) / THREADS;  // 16-byte pieces per thread
    static constexpr int kB = BN * (kBK / 8) / THREADS;
    u32x4 a[kA], b[kB];
};

template <int BM, int BN, int THREADS>
__device__ inline void tile_mma(const TileArgs& t, int k_begin, int k_end, uint16_t* lds,
                                f32x4 (&acc)[4][4]) {
    static_assert((BM / 64) * (BN / 64) * 64 == THREADS, "one wavefront per 64 x 64 block");
    using Regs = ChunkRegs<BM, BN, THREADS>;
    constexpr int MT = 4, NT = 4;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w / (BN / 64), wn = w % (BN / 64);
    uint16_t* la = lds;
    uint16_t* lb = lds + 2 * BM * kLdsK;
    const int nk = (k_end - k_begin) / kBK;
    // Chunks past the end reload the last one (never stored where it is read).
    auto gload = [&](Regs& R, int c) {
        const int k0 = k_begin + (c < nk ? c : nk - 1) * kBK;
#pragma unroll
        for (int i = 0; i < Regs::kA; ++i) {
            const int q = tid + THREADS * i;
            const int row = q >> 3, kc = (q & 7) * 8;
            R.a[i] = load16(t.A, t.m0 + row, t.K, k0 + kc, t.m0 + row < t.M);
        }
#pragma unroll
        for (int i = 0; i < Regs::kB; ++i) {
            const int q = tid + THREADS * i;
            const int row = q >> 3, kc = (q & 7) * 8;
            R.b[i] = load16(t.B, t.n0 + row, t.K, k0 + kc, t.n0 + row < t.Nc);
        }
    };
    auto lstore = [&](const Regs& R, int buf) {
#pragma unroll
        for (int i = 0; i < Regs::kA; ++i) {
            const int q = tid + THREADS * i;
            const int row = q >> 3, kc = (q & 7) * 8;
            *reinterpret_cast<u32x4*>(la + (buf * BM + row) * kLdsK + kc) = R.a[i];
        }
#pragma unroll
        for (int i = 0; i < Regs::kB; ++i) {
            const int q = tid + THREADS * i;
            const int row = q >> 3, kc = (q & 7) * 8;
            *reinterpret_cast<u32x4*>(lb + (buf * BN + row) * kLdsK + kc) = R.b[i];
        }
    };
    const int fr = lane & 15, fk = (lane >> 4) * 8;
    auto multiply = [&](int buf) {
#pragma unroll 1
        for (int ks = 0; ks < kBK; ks += 32) {
            bf16x8 a[MT], b[NT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                a[mt] = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(
                                la + (buf * BM + wm * 64 + mt * 16 + fr) * kLdsK + ks + fk));
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                b[nt] = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(
                                lb + (buf * BN + wn * 64 + nt * 16 + fr) * kLdsK + ks + fk));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[mt][nt] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt], b[nt], acc[mt][nt], 0, 0, 0);
        }
    };
    if (nk <= 0)
        return;
    Regs r0, r1;
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

template <int MT, int NT>
__device__ inline void zero(f32x4 (&acc)[MT][NT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            acc[mt][nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

// u[n][j] = bf16(sum_k h[n][k] w_down[j][k]): one workgroup of 16 wavefronts
// per TM x TN tile of u (rows x rank, 16 x 32, which keeps 256 workgroups at
// N = 256, r = 512). Wavefront w multiplies its own contiguous run of the K
// steps (32 wide), two steps per pass. A pass's 48 row segments (16 rows of
// h, 32 of W_down, 128 bytes each) are loaded row by row, eight rows per load
// instruction, two passes ahead into registers, then written to the
// wavefront's own LDS region (rows padded to 144 bytes, so a fragment read of
// 16 rows hits 16 different bank quads) and read back as MFMA fragments. A
// fragment loaded straight from memory touches 16 rows 8 KB apart per
// instruction, which ran at about half the rate. The 16 binary32 partial
// tiles are then added in wavefront order through LDS and rounded once, so no
// partial leaves the CU. Rows past N read row 0 and are not stored. The rank
// tile is the grid's fastest index: workgroups go to the XCDs in turn, so
// each XCD works on a few rank tiles and keeps their rows of W_down (with h)
// in its L2 instead of streaming all of W_down.
constexpr int kDownWaves = 16;
constexpr int kDownMT = 1, kDownNT = 2;
constexpr int kDownTM = 16 * kDownMT, kDownTN = 16 * kDownNT;
constexpr int kDownPass = 2;                           // K steps per pass
constexpr int kDownRows = kDownTM + kDownTN;           // row segments staged per pass
constexpr int kDownRowBytes = kDownPass * 32 * 2 + 16; // a segment and its padding
constexpr int kDownRowLanes = kDownPass * 32 * 2 / 16;  // lanes per row segment (16 bytes each)
constexpr int kDownRowsPerLoad = 64 / kDownRowLanes;    // segments per load instruction
constexpr int kDownLoads = kDownRows / kDownRowsPerLoad; // 16-byte loads per lane per pass
static_assert(kDownRows % kDownRowsPerLoad == 0 && kDownTM % kDownRowsPerLoad == 0, "whole loads");

__global__ __launch_bounds__(kDownWaves * 64) void head_down_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ w_down, int N, int r, int d,
    uint16_t* __restrict__ u) {
    __shared__ __align__(16) unsigned char stage[kDownWaves][kDownRows * kDownRowBytes];
    __shared__ float red[kDownWaves][kDownTM * kDownTN];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int m0 = static_cast<int>(blockIdx.y) * kDownTM;
    const int n0 = static_cast<int>(blockIdx.x) * kDownTN;
    const int steps = d / 32;
    const int per = (steps + kDownWaves - 1) / kDownWaves;
    const int s_begin = w * per < steps ? w * per : steps;
    const int s_end = s_begin + per < steps ? s_begin + per : steps;
    const int passes = (s_end - s_begin + kDownPass - 1) / kDownPass;
    // For load q, lane l loads 16 bytes of segment q * kDownRowsPerLoad + l /
    // kDownRowLanes, columns 8 (l % kDownRowLanes) on.
    const int sub = lane / kDownRowLanes, col = (lane % kDownRowLanes) * 8;
    unsigned char* region = stage[w];
    auto load_pass = [&](u32x4 (&R)[kDownLoads], int pass) {
        const int sa = s_begin + pass * kDownPass;
        const int sb = sa + kDownPass < s_end ? sa + kDownPass : s_end;
        const int kk = 32 * sa + col;
        const int k = kk < 32 * sb ? kk : 32 * s_begin + col;  // past the run: unused
#pragma unroll
        for (int q = 0; q < kDownLoads; ++q) {
            const int row = kDownRowsPerLoad * q + sub;
            const uint16_t* src;
            if (q < kDownTM / kDownRowsPerLoad) {
                const int hr = m0 + row;
                src = h + static_cast<size_t>(hr < N ? hr : 0) * d;
            } else {
                src = w_down + static_cast<size_t>(n0 + row - kDownTM) * d;
            }
            R[q] = *reinterpret_cast<const u32x4*>(src + k);
        }
    };
    f32x4 acc[kDownNT];
#pragma unroll
    for (int nt = 0; nt < kDownNT; ++nt)
        acc[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // Stage one pass's rows in the region and multiply its steps.
    auto run_pass = [&](const u32x4 (&R)[kDownLoads], int pass) {
#pragma unroll
        for (int q = 0; q < kDownLoads; ++q)
            *reinterpret_cast<u32x4*>(region + (kDownRowsPerLoad * q + sub) * kDownRowBytes +
                                      (lane % kDownRowLanes) * 16) = R[q];
        const int sa = s_begin + pass * kDownPass;
        const int frag = (lane & 15) * kDownRowBytes + (lane >> 4) * 16;
#pragma unroll
        for (int j = 0; j < kDownPass; ++j) {
            if (sa + j < s_end) {
                const bf16x8 a = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(region + frag + j * 64));
#pragma unroll
                for (int nt = 0; nt < kDownNT; ++nt) {
                    const bf16x8 b = __builtin_bit_cast(
                        bf16x8, *reinterpret_cast<const u32x4*>(
                                    region + (kDownTM + 16 * nt) * kDownRowBytes + frag + j * 64));
                    acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[nt], 0, 0, 0);
                }
            }
        }
    };
    // Two passes in flight: slot 0 holds the even passes, slot 1 the odd ones.
    u32x4 R0[kDownLoads], R1[kDownLoads];
    if (passes > 0)
        load_pass(R0, 0);
    if (passes > 1)
        load_pass(R1, 1);
    for (int pass = 0; pass < passes; pass += 2) {
        run_pass(R0, pass);
        if (pass + 2 < passes)
            load_pass(R0, pass + 2);
        if (pass + 1 < passes) {
            run_pass(R1, pass + 1);
            if (pass + 3 < passes)
                load_pass(R1, pass + 3);
        }
    }
    // Lane l holds C[4 (l / 16) + j][nt * 16 + l % 16] of the tile.
#pragma unroll
    for (int nt = 0; nt < kDownNT; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            red[w][(4 * (lane >> 4) + j) * kDownTN + nt * 16 + (lane & 15)] = acc[nt][j];
    __syncthreads();
    for (int t = threadIdx.x; t < kDownTM * kDownTN; t += kDownWaves * 64) {
        float sum = 0.0f;
#pragma unroll
        for (int q = 0; q < kDownWaves; ++q)
            sum += red[q][t];
        const int row = m0 + t / kDownTN, col_u = n0 + t % kDownTN;
        if (row < N)
            u[static_cast<size_t>(row) * r + col_u] = bf16_rne(sum);
    }
}


// z^T = bf16(W_up u^T) for one 128-vocabulary x 256-row tile, and each row's
// (m, s) over the tile's 128 vocabulary entries. Lane l of MFMA tile (mt, nt)
// holds logits v0..v0+3 (v0 = 4 * (l / 16) + ...) of row n = ... + l % 16, so
// the rounded logits go out as 8-byte stores of four consecutive entries, and
// a row's reduction runs over the lane's 16 values, the four lanes l % 16 + 16i
// (two shuffles) and the two wavefronts that share the row (through LDS).
__global__ __launch_bounds__(kUpThreads) void head_up_kernel(const uint16_t* __restrict__ u,
                                                           const uint16_t* __restrict__ w_up,
                                                           const float* __restrict__ temperature,
                                                           int N, int V, int r,
                                                           uint16_t* __restrict__ z,
                                                           HeadPart* __restrict__ part, int ntn) {
    constexpr int MT = 4, NT = 4;
    __shared__ __align__(16) uint16_t lds[lds_elems<kUpBM, kUpBN>()];
    __shared__ float lds_max[2][kUpBN];
    __shared__ double lds_sum[2][kUpBN];
    const int vt = static_cast<int>(blockIdx.x);
    const TileArgs t{w_up, u, V, N, r, vt * kUpBM, static_cast<int>(blockIdx.y) * kUpBN};
    f32x4 acc[MT][NT];
    zero(acc);
    tile_mma<kUpBM, kUpBN, kUpThreads>(t, 0, r, lds, acc);

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w / (kUpBN / 64), wn = w % (kUpBN / 64);
    const int vbase = t.m0 + wm * 64 + 4 * (lane >> 4);
    const int nloc0 = wn * 64 + (lane & 15);  // row within the tile, + 16 nt
    // Round to bf16, store, and keep the rounded values.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int n = t.n0 + nloc0 + nt * 16;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int v0 = vbase + mt * 16;
            uint16_t b[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                b[j] = bf16_rne(acc[mt][nt][j]);
                acc[mt][nt][j] = bf16_to_f32(b[j]);
            }
            if (n < N && v0 < V)  // V % 8 == 0: v0 < V covers all four
                *reinterpret_cast<uint2*>(z + static_cast<size_t>(n) * V + v0) =
                    make_uint2(b[0] | (static_cast<uint32_t>(b[1]) << 16),
                               b[2] | (static_cast<uint32_t>(b[3]) << 16));
        }
    }
    // Row maxima of x = fl32(z * fl32(1/T)) over the tile's valid entries.
    float inv_t[NT];
    bool act[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int n = t.n0 + nloc0 + nt * 16;
        inv_t[nt] = 0.0f;
        act[nt] = n < N && sampled_row(temperature[n < N ? n : 0], &inv_t[nt]);
        float xmax = -__builtin_huge_valf();
        if (act[nt]) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                if (vbase + mt * 16 < V)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        xmax = fmaxf(xmax, acc[mt][nt][j] * inv_t[nt]);
        }
        xmax = fmaxf(xmax, __shfl_xor(xmax, 16, 64));
        xmax = fmaxf(xmax, __shfl_xor(xmax, 32, 64));
        if (lane < 16)
            lds_max[wm][nloc0 + nt * 16] = xmax;
    }
    __syncthreads();
    // s = sum 2^(fma(x, log2e, -m)) with m = fl32(max x * log2e): eight terms
    // in binary32, then binary64.
    float m[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int nl = nloc0 + nt * 16;
        const float xmax = fmaxf(lds_max[0][nl], lds_max[1][nl]);
        m[nt] = xmax * kHeadLog2e;
        double sum = 0.0;
        if (act[nt] && xmax > -__builtin_huge_valf()) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                float g = 0.0f;
#pragma unroll
                for (int mt = 2 * half; mt < 2 * half + 2; ++mt)
                    if (vbase + mt * 16 < V)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            g += __builtin_amdgcn_exp2f(
                                __builtin_fmaf(acc[mt][nt][j] * inv_t[nt], kHeadLog2e, -m[nt]));
                sum += static_cast<double>(g);
            }
        }
        sum += __shfl_xor(sum, 16, 64);
        sum += __shfl_xor(sum, 32, 64);
        if (lane < 16)
            lds_sum[wm][nl] = sum;
    }
    __syncthreads();
    if (wm == 0 && lane < 16) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int nl = nloc0 + nt * 16;
            const int n = t.n0 + nl;
            if (n < N)
                part[static_cast<size_t>(n) * ntn + vt] =
                    HeadPart{m[nt], 0, lds_sum[0][nl] + lds_sum[1][nl]};
        }
    }
}

// Streaming form of the second product for rank r = 32 * KS, KS in {8, 16}.
// Each of the G workgroups (one per CU) owns a contiguous run of 16-row
// blocks of W_up and all of a 256-row batch tile:
// * every wavefront keeps the B fragments of its 32 batch rows (all of K) in
//   registers for the whole run (each W_up fragment read from LDS feeds two
//   matrix instructions; 64 rows per wavefront would halve the LDS reads but
//   leave one wavefront per SIMD, which measured slower);
// * blocks of W_up stream through a ring of kRing LDS slots, loaded straight
//   into LDS kRing - 1 blocks ahead, one or two whole rows per load (a load
//   of MFMA fragments would touch 16 rows per instruction, which measured
//   slower); a row's 16-byte chunks are stored at positions XORed with the
//   row number, so a fragment read (16 rows, one chunk each) hits 16
//   different bank quads;
// * each block gives every wavefront a 16 x 32 piece of z^T, rounded and
//   stored as 8-byte runs, and folded into per-row (m, s) pairs online: when a
//   block raises a row's maximum the pair is rescaled by a binary32 exp2
//   factor, and each block adds at most four binary32 terms to the binary64 s;
// * a step multiplies block b out while it rounds, stores and folds block
//   b - 1, so matrix and vector instructions interleave.
// The pieces of the four lanes sharing a row are merged at the end into one
// (m, s) per (row, workgroup).
constexpr int kRing = 6;
constexpr int kStreamWaves = 8;   // two per SIMD, so one's matrix work covers the other's waits
constexpr int kStreamRows = 32;

__device__ constexpr int vmcnt_imm(int n) {
    // s_waitcnt operand: vmcnt n (bits 3:0 and 15:14), expcnt and lgkmcnt not waited
    return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

template <int KS>
__global__ __launch_bounds__(kStreamWaves * 64) void head_up_stream_kernel(
    const uint16_t* __restrict__ u, const uint16_t* __restrict__ w_up,
    const float* __restrict__ temperature, int N, int V, uint16_t* __restrict__ z,
    HeadPart* __restrict__ part, int nparts, uint2* __restrict__ sink) {
    static_assert(KS % kStreamWaves == 0, "each wavefront loads KS / 8 fragments per block");
    constexpr int NT = kStreamRows / 16;
    constexpr int K = KS * 32;
    constexpr int kLoadsPerBlock = KS / kStreamWaves;  // per wavefront
    constexpr int kChunks = KS * 4;                    // 16-byte chunks of a W_up row
    constexpr int kRowsPerLoad = 64 / kChunks;         // rows of a block one load covers
    static_assert(kChunks % 16 == 0 && 64 % kChunks == 0, "whole rows per load, 16 bank quads per row");
    __shared__ __align__(16) uint16_t ring[kRing][KS * 512];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int g = blockIdx.x, G = gridDim.x;
    const int nblk = (V + 15) / 16;
    const int b0 = static_cast<int>(static_cast<long>(nblk) * g / G);
    const int b1 = static_cast<int>(static_cast<long>(nblk) * (g + 1) / G);
    const int n0 = static_cast<int>(blockIdx.y) * (kStreamWaves * kStreamRows) + wv * kStreamRows;

    // Block b into slot (b - b0) % kRing. Blocks past the run reload the run's
    // last block into a slot nobody reads again: every wavefront always issues
    // kLoadsPerBlock loads per step, which the waits below count on.
    auto issue = [&](int b) {
        const int bb = b < b1 ? b : b1 - 1;
        uint16_t* slot = ring[(b - b0) % kRing];
#pragma unroll
        for (int i = 0; i < kLoadsPerBlock; ++i) {
            // Load ks covers rows ks * kRowsPerLoad ...: each lane one 16-byte
            // chunk, the row's chunk (position ^ row) at the lane's position.
            const int ks = wv + kStreamWaves * i;
            const int row = ks * kRowsPerLoad + lane / kChunks;
            const int v = bb * 16 + row;
            const uint16_t* src = w_up + static_cast<size_t>(v < V ? v : V - 1) * K +
                                  ((lane % kChunks) ^ row) * 8;
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src), slot + ks * 512, 16,
                                             0, 0);
        }
    };
    float inv_t[NT], mref[NT];
    double sacc[NT];
    bool act[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int n = n0 + nt * 16 + (lane & 15);
        inv_t[nt] = 0.0f;
        act[nt] = n < N && sampled_row(temperature[n < N ? n : 0], &inv_t[nt]);
        mref[nt] = -__builtin_huge_valf();
        sacc[nt] = 0.0;
    }

    // This wavefront's batch rows as B fragments (rows past N read row 0).
    bf16x8 ub[NT][KS];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int n = n0 + nt * 16 + (lane & 15);
        const uint16_t* urow = u + static_cast<size_t>(n < N ? n : 0) * K + (lane >> 4) * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            ub[nt][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(urow + ks * 32));
    }
    // The first kRing - 1 blocks; the temperature and U loads above are
    // older, so the step waits below cover them too.
#pragma unroll
    for (int i = 0; i < kRing - 1; ++i)
        issue(b0 + i);
    // Left alone, the compiler moves the U loads below the first barrier,
    // next to their first use, so the kernel start takes two memory round
    // trips (ring, then U). Naming the registers here keeps all of them in
    // flight together.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            asm volatile("" : "+v"(ub[nt][ks]));

    // Finishing block b: lane l holds logits v0..v0+3 of row n (V % 8 == 0:
    // v0 < V covers all four). Part 2 nt rounds and scales row tile nt and
    // moves its reference; part 2 nt + 1 adds its terms and stores it. Lanes
    // outside the batch or the vocabulary store to their own word of a sink:
    // no branch anywhere, so the parts can sit between matrix instructions.
    float fx[NT][4], fscale[NT];
    uint2 fpack[NT];
    auto finish = [&](int b, const f32x4 (&acc)[NT], int part) {
        const int nt = part >> 1;
        const int v0 = b * 16 + 4 * (lane >> 4);
        const bool on = act[nt] && v0 < V;
        if ((part & 1) == 0) {
            // Two logits per conversion instruction, rounded to nearest even
            // (the low element in the low half).
            const uint32_t w0 = __builtin_bit_cast(
                uint32_t, __builtin_convertvector(f32x2{acc[nt][0], acc[nt][1]}, bf16x2));
            const uint32_t w1 = __builtin_bit_cast(
                uint32_t, __builtin_convertvector(f32x2{acc[nt][2], acc[nt][3]}, bf16x2));
            fx[nt][0] = __uint_as_float(w0 << 16) * inv_t[nt];
            fx[nt][1] = __uint_as_float(w0 & 0xFFFF0000u) * inv_t[nt];
            fx[nt][2] = __uint_as_float(w1 << 16) * inv_t[nt];
            fx[nt][3] = __uint_as_float(w1 & 0xFFFF0000u) * inv_t[nt];
            fpack[nt] = make_uint2(w0, w1);
            const float bm = on ? fmaxf(fmaxf(fx[nt][0], fx[nt][1]), fmaxf(fx[nt][2], fx[nt][3]))
                                : -__builtin_huge_valf();
            const float m_new = fmaxf(mref[nt], bm * kHeadLog2e);  // fl32(max x * log2e)
            fscale[nt] = mref[nt] == m_new ? 1.0f : __builtin_amdgcn_exp2f(mref[nt] - m_new);
            mref[nt] = m_new;
        } else {
            const bool live = on && mref[nt] > -__builtin_huge_valf();
            float gsum = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(fx[nt][j], kHeadLog2e, -mref[nt]));
                gsum += live ? e : 0.0f;
            }
            sacc[nt] = sacc[nt] * static_cast<double>(fscale[nt]) + static_cast<double>(gsum);
            const int n = n0 + nt * 16 + (lane & 15);
            uint2* dst = n < N && v0 < V
                             ? reinterpret_cast<uint2*>(z + static_cast<size_t>(n) * V + v0)
                             : sink + lane;
            *dst = fpack[nt];
        }
    };
    static_assert(2 * NT == 4, "four finishing parts, one per quarter of K");
    // Fragments one quarter of K ahead: while the matrix instructions of
    // quarter q of block b run, the four fragments of the next quarter (of
    // block b, or quarter 0 of block b + 1) are read from LDS into the other
    // half of a two-quarter register buffer, so the reads hide behind the
    // matrix work instead of preceding it.
    constexpr int QK = KS / 4;  // fragments per quarter
    auto read_quarter = [&](int b, int q, bf16x8 (&a)[QK]) {
        const uint16_t* slot = ring[(b - b0) % kRing];
        const int r = lane & 15;
#pragma unroll
        for (int i = 0; i < QK; ++i) {
            // Row r's chunk c of fragment ks sits at position c ^ r of the row.
            const int c = 4 * (q * QK + i) + (lane >> 4);
            a[i] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(slot + (r * kChunks + (c ^ r)) * 8));
        }
    };
    auto mma_q = [&](const bf16x8 (&a)[QK], f32x4 (&acc)[NT], int q) {
#pragma unroll
        for (int i = 0; i < QK; ++i)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], ub[nt][q * QK + i], acc[nt],
                                                                  0, 0, 0);
    };
    // Block b + 1 is readable once its loads have landed (loads complete in
    // order, and kLoadsPerBlock * (kRing - 3) loads were issued after them:
    // stores issued meanwhile only make this wait stricter) and the barrier
    // has made every wavefront's part visible. Passing the barrier also means
    // every wavefront has finished block b - 1, whose slot is refilled next.
    auto publish_next = [&](int b) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoadsPerBlock * (kRing - 3)));
        __syncthreads();
        issue(b + kRing - 1);
    };
    // Block b0 first: its loads are followed by kRing - 2 blocks' worth.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoadsPerBlock * (kRing - 2)));
    __syncthreads();
    bf16x8 qa[2][QK];
    read_quarter(b0, 0, qa[0]);
    // Two-stage pipeline: block b is multiplied while block b - 1 is finished,
    // a quarter of each at a time, and the next quarter's fragments are read.
    f32x4 acc_c[NT], acc_n[NT];
    for (int b = b0; b < b1; ++b) {
        publish_next(b);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            acc_n[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (q < 3)
                read_quarter(b, q + 1, qa[(q + 1) & 1]);
            else
                read_quarter(b + 1, 0, qa[0]);  // past the run: the reloaded last block, unused
            mma_q(qa[q & 1], acc_n, q);
            if (b > b0)
                finish(b - 1, acc_c, q);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            acc_c[nt] = acc_n[nt];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
        finish(b1 - 1, acc_c, q);
    // The last steps' ring loads land in slots nobody reads; drain them so no
    // write into this workgroup's LDS is pending when the workgroup ends.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    // Merge the four lanes of each row (l % 16 + 16 i), then one piece per row.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int off = 16; off < 64; off <<= 1) {
            const float mo = __shfl_xor(mref[nt], off, 64);
            const double so = __shfl_xor(sacc[nt], off, 64);
            const float mn = fmaxf(mref[nt], mo);
            const double a = sacc[nt] == 0.0 ? 0.0
                             : mref[nt] == mn ? sacc[nt]
                                              : sacc[nt] * static_cast<double>(__builtin_amdgcn_exp2f(mref[nt] - mn));
            const double c = so == 0.0 ? 0.0
                             : mo == mn ? so : so * static_cast<double>(__builtin_amdgcn_exp2f(mo - mn));
            mref[nt] = mn;
            sacc[nt] = a + c;
        }
        const int n = n0 + nt * 16 + lane;
        if (lane < 16 && n < N)
            part[static_cast<size_t>(n) * nparts + g] = HeadPart{mref[nt], 0, sacc[nt]};
    }
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
    int ntn = 0;
    int stream_groups = 0;  // > 0: the streaming second product with this many workgroups
    hipStream_t stream = nullptr;
    void* ws = nullptr;
    uint16_t* u = nullptr;
    HeadPart* part = nullptr;
    uint2* sink = nullptr;  // 64 words the streaming kernel's idle lanes store to
};

extern "C" {

int spec_lowrank_head_init(int rows, int hidden, int rank, int vocab, void* hip_stream,
                           spec_head_ctx** out_ctx) {
    if (!out_ctx)
        return SPEC_EINVAL;
    *out_ctx = nullptr;
    if (rows < 1 || hidden < kBK || hidden % kBK || rank < kBK || rank % kBK || vocab < 8 ||
        vocab % 8 || (rows + kDownTM - 1) / kDownTM > 65535)
        return SPEC_EINVAL;
    spec_head_ctx* ctx = new (std::nothrow) spec_head_ctx();
    if (!ctx)
        return SPEC_ENOMEM;
    ctx->N = rows;
    ctx->d = hidden;
    ctx->r = rank;
    ctx->V = vocab;
    ctx->stream = static_cast<hipStream_t>(hip_stream);
    ctx->ntn = (vocab + kUpBM - 1) / kUpBM;
    if (rank == 256 || rank == 512) {
        // One workgroup per CU, each with at least one 16-row block of W_up.
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus < 1) {
            delete ctx;
            return SPEC_EHIP;
        }
        ctx->stream_groups = std::min(cus, (vocab + 15) / 16);
        ctx->ntn = ctx->stream_groups;
    }
    const size_t nr = static_cast<size_t>(rows) * rank;
    size_t off = 0;
    const size_t o_u = off;
    off = align_up(off + nr * sizeof(uint16_t), 256);
    const size_t o_h = off;
    off = align_up(off + static_cast<size_t>(rows) * ctx->ntn * sizeof(HeadPart), 256);
    const size_t o_s = off;
    off = align_up(off + 64 * sizeof(uint2), 256);
    if (hipMalloc(&ctx->ws, off) != hipSuccess) {
        delete ctx;
        return SPEC_ENOMEM;
    }
    char* base = static_cast<char*>(ctx->ws);
    ctx->u = reinterpret_cast<uint16_t*>(base + o_u);
    ctx->part = reinterpret_cast<HeadPart*>(base + o_h);
    ctx->sink = reinterpret_cast<uint2*>(base + o_s);
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
    head_down_kernel<<<dim3(static_cast<unsigned>(r / kDownTN),
                            static_cast<unsigned>((N + kDownTM - 1) / kDownTM)),
                       dim3(kDownWaves * 64), 0, s>>>(static_cast<const uint16_t*>(hidden),
                                                      static_cast<const uint16_t*>(w_down), N, r,
                                                      d, ctx->u);
    if (hipGetLastError() != hipSuccess)
        return SPEC_EHIP;
    if (ctx->stream_groups > 0) {
        const dim3 grid(static_cast<unsigned>(ctx->stream_groups),
                        static_cast<unsigned>((N + kStreamWaves * kStreamRows - 1) / (kStreamWaves * kStreamRows)));
        if (r == 512)
            head_up_stream_kernel<16><<<grid, dim3(kStreamWaves * 64), 0, s>>>(
                ctx->u, static_cast<const uint16_t*>(w_up), temperature, N, V,
                static_cast<uint16_t*>(out_logits), ctx->part, ctx->ntn, ctx->sink);
        else
            head_up_stream_kernel<8><<<grid, dim3(kStreamWaves * 64), 0, s>>>(
                ctx->u, static_cast<const uint16_t*>(w_up), temperature, N, V,
                static_cast<uint16_t*>(out_logits), ctx->part, ctx->ntn, ctx->sink);
    } else {
        head_up_kernel<<<dim3(static_cast<unsigned>(ctx->ntn), static_cast<unsigned>((N + kUpBN - 1) / kUpBN)),
                         dim3(kUpThreads), 0, s>>>(
            ctx->u, static_cast<const uint16_t*>(w_up), temperature, N, V, r,
            static_cast<uint16_t*>(out_logits), ctx->part, ctx->ntn);
    }
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
