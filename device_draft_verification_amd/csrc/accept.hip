// Accept kernel: one 64-lane wavefront per sequence runs the accept step of
// accept.hpp (split merge, gather, log-space test, first rejection, emitted
// prefix) and leaves (k, u_res) and the row coefficients for the draw. The
// verification outcome -- accepted count plus the extra token -- is what the
// Speculative Speculative Decoding summary (section 2, central concept, item
// 1) keys its speculation cache on.
//
// Also here: the scalar-only accept (O(B * gamma) bytes, nothing of size V)
// and the Philox test export.
#include <math.h>

#include "accept.hpp"

namespace specv {
namespace {

__global__ __launch_bounds__(64) void accept_kernel(AcceptArgs a) {
    (void)accept_sequence(a, blockIdx.x, true);
}

__global__ __launch_bounds__(256) void accept_scalar_kernel(const float* __restrict__ logprobs,
                                                            int batch, int gamma, uint64_t seed,
                                                            uint64_t offset,
                                                            int32_t* __restrict__ out_len) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= batch)
        return;
    int k = gamma;
    for (int i = 0; i < gamma; ++i) {
        const float2 pr = reinterpret_cast<const float2*>(logprobs)[static_cast<size_t>(b) * gamma + i];
        const double d = static_cast<double>(pr.y) - static_cast<double>(pr.x);
        const Words4 w = verify_block(seed, offset, static_cast<uint32_t>(b), static_cast<uint32_t>(i));
        const double log_u = log(static_cast<double>(uniform24(w.w0)));
        if (!(log_u < d)) {
            k = i;
            break;
        }
    }
    out_len[b] = k;
}

__global__ __launch_bounds__(256) void philox_words_kernel(int batch, int gamma, uint64_t seed,
                                                           uint64_t offset, uint32_t* __restrict__ out) {
    const long n = static_cast<long>(batch) * (gamma + 1);
    const long t = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= n)
        return;
    const uint32_t b = static_cast<uint32_t>(t / (gamma + 1));
    const uint32_t i = static_cast<uint32_t>(t % (gamma + 1));
    const Words4 w = verify_block(seed, offset, b, i);
    reinterpret_cast<uint4*>(out)[t] = make_uint4(w.w0, w.w1, w.w2, w.w3);
}

}  // namespace

hipError_t launch_accept(int batch, const AcceptArgs& a, hipStream_t stream,
                         const LaunchEvents& ev) {
    if (batch == 0)
        return hipSuccess;
    return launch(accept_kernel, dim3(batch), dim3(64), 0, stream, ev, a);
}

hipError_t launch_accept_scalar(int batch, int gamma, const float* logprobs, uint64_t seed,
                                uint64_t offset, int32_t* out_len, hipStream_t stream) {
    if (batch == 0)
        return hipSuccess;
    const int blocks = (batch + 255) / 256;
    accept_scalar_kernel<<<dim3(blocks), dim3(256), 0, stream>>>(logprobs, batch, gamma, seed,
                                                                 offset, out_len);
    return hipGetLastError();
}

hipError_t launch_philox_words(int batch, int gamma, uint64_t seed, uint64_t offset,
                               uint32_t* out, hipStream_t stream) {
    const long n = static_cast<long>(batch) * (gamma + 1);
    if (n == 0)
        return hipSuccess;
    const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
    philox_words_kernel<<<dim3(blocks), dim3(256), 0, stream>>>(batch, gamma, seed, offset, out);
    return hipGetLastError();
}

}  // namespace specv
