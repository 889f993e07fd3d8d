// Shared device-side definitions of the verification kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specv {

constexpr int kBlock = 256;        // threads per workgroup of the vocabulary kernels
constexpr int kWaves = kBlock / 64;
constexpr int kMaxSplit = 64;     // most vocabulary splits of one row
// log2(e) rounded to binary32. Row normalisers are kept in base-2 units of this
// constant: s = sum_v 2^(x_v * kLog2e - m), lse = (m + log2 s) / kLog2e, which is
// the natural log-sum-exp of x up to a relative change of 1.3e-8 in the scale
// of x (the rounding of the constant), i.e. below 2e-7 absolute for any row.
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kNegMax = -3.402823466e38f;   // "no finite entry yet" reference

enum Dtype { kF32 = 0, kBF16 = 1 };

// Per (row, vocabulary split) result of the row kernel. Sampling rows: m is the
// base-2 reference max(x) * kLog2e rounded to binary32 and s = sum 2^(x*kLog2e - m)
// over the split. Greedy rows: m is the largest raw logit and idx its lowest index.
struct Partial {
    float m;
    int idx;
    double s;
};

// A whole row after the splits are merged (same meaning as Partial).
struct RowNorm {
    float m;
    int idx;
    double s;
};

// What the accept kernel leaves for the residual kernels, per sequence: the
// outcome and every coefficient they need, so their prologue is one load.
struct SeqState {
    int k;        // first rejected position, or gamma
    int mode;     // 1: draw the extra token from the residual / bonus row
    float u_res;  // resample uniform of position k
    float inv_t;  // fl32(1 / T)
    float mp;     // base-2 reference of target row k
    float mq;     // base-2 reference of draft row k (k < gamma)
    float ratio;  // s_q / s_p of those rows (k < gamma), else 1
    int pad;
};

// ---------------------------------------------------------------- loading ---

// A "group" is what one 16-byte load brings: 8 bf16 or 4 fp32 logits. When the
// rows are not 16-byte aligned the kernels fall back to groups of one element.
template <int DT, bool VEC>
struct Group {
    static constexpr int W = VEC ? (DT == kBF16 ? 8 : 4) : 1;
};

template <int DT, bool VEC>
struct Loader {
    static constexpr int W = Group<DT, VEC>::W;
    using raw_t = typename std::conditional<VEC, uint4,
                  typename std::conditional<DT == kBF16, uint16_t, float>::type>::type;

    __device__ static inline raw_t load(const void* row, long g) {
        return reinterpret_cast<const raw_t*>(row)[g];
    }

    // Streaming load: marked non-temporal so it does not displace reusable lines.
    __device__ static inline raw_t load_nt(const void* row, long g) {
        if constexpr (VEC) {
            typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row) + g);
            return make_uint4(v.x, v.y, v.z, v.w);
        } else {
            return __builtin_nontemporal_load(reinterpret_cast<const raw_t*>(row) + g);
        }
    }

    // A group of -inf logits (the identity of max and of sum-of-exp).
    __device__ static inline raw_t neg_inf() {
        if constexpr (VEC) {
            const unsigned w = DT == kBF16 ? 0xFF80FF80u : 0xFF800000u;
            return make_uint4(w, w, w, w);
        } else if constexpr (DT == kBF16) {
            return static_cast<uint16_t>(0xFF80u);
        } else {
            return -__builtin_huge_valf();
        }
    }

    template <bool NT>
    __device__ static inline raw_t load_as(const void* row, long g) {
        if constexpr (NT)
            return load_nt(row, g);
        else
            return load(row, g);
    }

    __device__ static inline void unpack(const raw_t& q, float (&z)[W]) {
        if constexpr (VEC) {
            if constexpr (DT == kBF16) {
                const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    z[2 * i] = __uint_as_float(w[i] << 16);
                    z[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
                }
            } else {
                z[0] = __uint_as_float(q.x);
                z[1] = __uint_as_float(q.y);
                z[2] = __uint_as_float(q.z);
                z[3] = __uint_as_float(q.w);
            }
        } else {
            if constexpr (DT == kBF16)
                z[0] = __uint_as_float(static_cast<uint32_t>(q) << 16);
            else
                z[0] = q;
        }
    }
};

__device__ inline float load_logit(const void* row, int dtype, long v) {
    if (dtype == kBF16)
        return __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(row)[v]) << 16);
    return reinterpret_cast<const float*>(row)[v];
}

// The same logit as raw bits (bf16 in the low half, or fp32), and its value:
// a load whose conversion is left for later is waited for only there.
__device__ inline uint32_t load_logit_bits(const void* row, int dtype, long v) {
    if (dtype == kBF16)
        return static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(row)[v]);
    return reinterpret_cast<const uint32_t*>(row)[v];
}

__device__ inline float logit_of_bits(uint32_t bits, int dtype) {
    return __uint_as_float(dtype == kBF16 ? bits << 16 : bits);
}

__device__ inline const void* row_ptr(const void* base, int dtype, size_t row, int vocab) {
    const size_t esz = dtype == kBF16 ? 2 : 4;
    return static_cast<const char*>(base) + row * static_cast<size_t>(vocab) * esz;
}

// ------------------------------------------------------------ arithmetic ---

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x = fl32(z * inv_t): one binary32 multiply (contraction is off in this library).
__device__ inline float scale_logit(float z, float inv_t) { return z * inv_t; }

// ------------------------------------------------------ wave/block helpers ---

__device__ inline float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ inline double wave_sum(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// Block max / sum over kBlock threads, result broadcast to all threads.
// Deterministic: a fixed butterfly per wave, then waves combined in order.
__device__ inline float block_max(float v, float* lds) {
    v = wave_max(v);
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();
    if (lane == 0)
        lds[wid] = v;
    __syncthreads();
    float r = lds[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w)
        r = fmaxf(r, lds[w]);
    return r;
}

__device__ inline double block_sum(double v, double* lds) {
    v = wave_sum(v);
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();
    if (lane == 0)
        lds[wid] = v;
    __syncthreads();
    double r = lds[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w)
        r += lds[w];
    return r;
}

// Exclusive prefix sum over the block in thread order; *total gets the sum.
__device__ inline double block_exclusive_scan(double v, double* lds, double* total) {
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    double inc = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(inc, off, 64);
        if (lane >= off)
            inc += o;
    }
    __syncthreads();
    if (lane == 63)
        lds[wid] = inc;
    __syncthreads();
    double before = 0.0, all = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        if (w < wid)
            before += lds[w];
        all += lds[w];
    }
    *total = all;
    return before + inc - v;
}

// Lowest thread index whose flag is set, or kBlock if none.
__device__ inline int block_first(bool flag, int* lds) {
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const unsigned long long m = __ballot(flag);
    __syncthreads();
    if (lane == 0)
        lds[wid] = m ? wid * 64 + __ffsll(static_cast<long long>(m)) - 1 : kBlock;
    __syncthreads();
    int r = kBlock;
#pragma unroll
    for (int w = kWaves - 1; w >= 0; --w)
        r = lds[w] < kBlock ? lds[w] : r;
    return r;
}

__device__ inline int block_max_int(int v, int* lds) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const int o = __shfl_xor(v, off, 64);
        v = o > v ? o : v;
    }
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();
    if (lane == 0)
        lds[wid] = v;
    __syncthreads();
    int r = lds[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w)
        r = lds[w] > r ? lds[w] : r;
    return r;
}

// Vocabulary split c of n over `groups` groups: [begin, end).
__device__ inline void split_range(long groups, int n, int c, long* begin, long* end) {
    const long per = (groups + n - 1) / n;
    long b = per * c, e = b + per;
    if (b > groups) b = groups;
    if (e > groups) e = groups;
    *begin = b;
    *end = e;
}

}  // namespace specv
