// Philox4x32-10 counter-based generator for the device.
//
// Written from its published definition (Salmon, Moraes, Dror and Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC'11): ten rounds of the
// Philox S-box on a 128-bit counter under a 64-bit key. A round multiplies
// counter words 0 and 2 by two odd 32-bit multipliers into 64-bit products and
// forms (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)); the key
// is bumped by two Weyl constants between rounds.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specv {

struct Words4 {
    uint32_t w0, w1, w2, w3;
};

__device__ inline Words4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                       uint32_t k0, uint32_t k1) {
    constexpr uint32_t kMulA = 0xD2511F53u;
    constexpr uint32_t kMulB = 0xCD9E8D57u;
    constexpr uint32_t kWeylA = 0x9E3779B9u;
    constexpr uint32_t kWeylB = 0xBB67AE85u;
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint32_t lo_a = kMulA * c0, hi_a = __umulhi(kMulA, c0);
        const uint32_t lo_b = kMulB * c2, hi_b = __umulhi(kMulB, c2);
        const uint32_t n0 = hi_b ^ c1 ^ k0;
        const uint32_t n2 = hi_a ^ c3 ^ k1;
        c0 = n0;
        c1 = lo_b;
        c2 = n2;
        c3 = lo_a;
        k0 += kWeylA;
        k1 += kWeylB;
    }
    return Words4{c0, c1, c2, c3};
}

// The block of (sequence b, position i) for a call's (seed, offset): key
// (lo32 seed, hi32 seed), counter (i, b, lo32 offset, hi32 offset).
__device__ inline Words4 verify_block(uint64_t seed, uint64_t offset, uint32_t b, uint32_t i) {
    return philox4x32_10(i, b, static_cast<uint32_t>(offset), static_cast<uint32_t>(offset >> 32),
                         static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
}

// 24-bit uniform in [0, 1): the top 24 bits of a word times 2^-24 (exact in fp32).
__device__ inline float uniform24(uint32_t w) {
    return static_cast<float>(w >> 8) * (1.0f / 16777216.0f);
}

}  // namespace specv
