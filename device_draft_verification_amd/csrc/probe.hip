// Read-only HBM probe: the practical ceiling the streaming kernels are
// measured against, beside the vendor peak. The buffer is cut into one
// contiguous run per workgroup (the row kernel's pattern); each thread streams
// 16-byte non-temporal loads at a stride of the workgroup, eight in flight,
// folds them with xor so nothing is optimised away, and each workgroup leaves
// one word in a sink. Nothing is computed per byte beyond the xor, so the
// kernel's duration is the time HBM takes to deliver the buffer.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spec_verify.h"

namespace {

constexpr int kProbeBlock = 256;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeBlock) void hbm_read_probe_kernel(const uint4* __restrict__ buf,
                                                                     uint64_t n16,
                                                                     uint32_t* __restrict__ sink) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4* p = reinterpret_cast<const u32x4*>(buf);
    // this workgroup's run [a, e) of 16-byte words
    const uint64_t a = n16 * blockIdx.x / gridDim.x;
    const uint64_t e = n16 * (blockIdx.x + 1) / gridDim.x;
    uint64_t i = a + threadIdx.x;
    uint32_t acc = 0;
    // Two batches of kProbeUnroll loads in flight: the next batch is issued
    // before the current one is folded. Loads past the run read its first
    // word (in bounds) and are not folded.
    constexpr uint64_t kBatch = static_cast<uint64_t>(kProbeUnroll) * kProbeBlock;
    auto load_batch = [&](u32x4 (&v)[kProbeUnroll], uint64_t base) {
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const uint64_t j = base + static_cast<uint64_t>(u) * kProbeBlock;
            v[u] = __builtin_nontemporal_load(p + (j < e ? j : a));
        }
    };
    auto fold = [&](const u32x4 (&v)[kProbeUnroll], uint64_t base) {
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u)
            if (base + static_cast<uint64_t>(u) * kProbeBlock < e)
                acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    };
    u32x4 va[kProbeUnroll], vb[kProbeUnroll];
    load_batch(va, i);
    while (i < e) {
        load_batch(vb, i + kBatch);
        fold(va, i);
        i += kBatch;
        if (i >= e)
            break;
        load_batch(va, i + kBatch);
        fold(vb, i);
        i += kBatch;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), off, 64));
    __shared__ uint32_t part[kProbeBlock / 64];
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0)
        sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

extern "C" int spec_hbm_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, int blocks,
                                   void* hip_stream) {
    if (!buf || !sink || blocks < 1 || bytes % 16 != 0 ||
        reinterpret_cast<uintptr_t>(buf) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
        return SPEC_EINVAL;
    if (bytes == 0)
        return SPEC_OK;
    hbm_read_probe_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(kProbeBlock), 0,
                            static_cast<hipStream_t>(hip_stream)>>>(
        static_cast<const uint4*>(buf), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}
