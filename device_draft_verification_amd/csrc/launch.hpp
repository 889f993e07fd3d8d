// Host-side launchers of the verification kernels (one per translation unit).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

#include "common.hpp"

namespace specv {

// Temperature classification shared by the kernels: -1 invalid, 0 greedy, 1 sampled.
__device__ inline int temperature_mode(float t, float* inv_t) {
    if (!(t >= 0.0f) || t == __builtin_huge_valf())
        return -1;
    if (t == 0.0f) {
        *inv_t = 0.0f;
        return 0;
    }
    const float r = 1.0f / t;  // correctly rounded binary32 division
    if (r == __builtin_huge_valf())
        return -1;
    *inv_t = r;
    return 1;
}

struct Shape {
    int batch, gamma, vocab, dtype;
};

// Start and stop events of a launch in timing mode. They are attached to the
// kernel's own dispatch (hipExtLaunchKernel), so their interval is the kernel
// alone, with no marker packet of its own between kernels. Both null: a
// plain launch.
struct LaunchEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

template <typename... Params, typename... Args>
inline hipError_t launch(void (*kern)(Params...), dim3 grid, dim3 block, size_t shmem,
                         hipStream_t stream, const LaunchEvents& ev, Args... args) {
    static_assert(sizeof...(Params) == sizeof...(Args), "one argument per kernel parameter");
    if (!ev.start && !ev.stop) {
        kern<<<grid, block, shmem, stream>>>(args...);
        return hipGetLastError();
    }
    std::tuple<Params...> vals{static_cast<Params>(args)...};
    void* ptrs[sizeof...(Params) > 0 ? sizeof...(Params) : 1];
    std::apply([&](auto&... v) {
        size_t i = 0;
        ((ptrs[i++] = static_cast<void*>(&v)), ...);
    }, vals);
    return hipExtLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, ptrs,
                              shmem, stream, ev.start, ev.stop, 0);
}

// Launch geometry of the row-normaliser kernel.
struct RowTuning {
    int nsplit;        // vocabulary splits per row
    int unroll;        // 16-byte groups in flight per thread: 2, 4 or 8
    bool nontemporal;  // streaming loads marked non-temporal
};

// Row normalisers: grid = B * (2G+1) * nsplit workgroups of kBlock threads.
// Also records, per row of a position i < G, the raw logit of draft token t_i
// in gathered[row] (rows of invalid tokens are left untouched).
hipError_t launch_row_norm(const Shape& s, bool vec, const RowTuning& tu, const void* draft,
                           const void* target, const float* temperature, const int32_t* tokens,
                           Partial* part, float* gathered, hipStream_t stream,
                           const LaunchEvents& ev = LaunchEvents{});

// Everything the accept step reads and writes.
struct AcceptArgs {
    const int32_t* tokens;
    const float* temperature;
    int gamma, vocab, nsplit;  // nsplit: vocabulary splits of the row kernel
    uint64_t seed, offset;
    const uint64_t* offset_dev;  // non-null: the Philox offset is this device word
    const Partial* part;
    const float* gathered;
    RowNorm* rn;
    double* lse_out;
    SeqState* seq;
    int32_t* out_len;
    int32_t* out_tok;
};

// Split merge, gather, accept test, first rejection and the emitted prefix:
// one 64-lane wavefront per sequence. With offset_dev non-null the Philox
// offset is read from that device word instead of `offset`.
hipError_t launch_accept(int batch, const AcceptArgs& a, hipStream_t stream,
                         const LaunchEvents& ev = LaunchEvents{});

// Residual / bonus draw at the first rejection: per-tile sums (B * nsplit
// workgroups, `unroll` tiles per batch per wavefront: 2 or 4), then one
// locating wavefront per sequence. tile_sums holds
// B * residual_tiles_per_row(vocab) floats. nsplit == 0 selects the fused
// kernel instead (one workgroup per sequence, tile sums in LDS, one launch),
// for rows of at most residual_fused_max_tiles() tiles. With acc non-null
// (tile path only) the tile kernel also runs the accept step, split 0 writing
// its outputs, so no accept launch precedes it.
int residual_tiles_per_row(int vocab);
int residual_fused_max_tiles();
hipError_t launch_residual(const Shape& s, bool vec, int nsplit, int unroll, const void* draft,
                           const void* target, const SeqState* seq, float* tile_sums,
                           int32_t* out_tok, const AcceptArgs* acc, hipStream_t stream,
                           const LaunchEvents& ev = LaunchEvents{});

// Sampled verification of draft trees (spec_tree.h): each tree split over
// tree_sample_parts() workgroups, n_groups trees at a time (at most
// tree_sample_max_groups, which the device holds at once). shares holds
// n_groups * tree_sample_group_bytes() bytes and ctl three 64-bit words
// (launches finished, workgroups finished in the running launch, trees given
// up), all zeroed once before the first call and kept by the kernel itself
// from then on. A part gives up on a partner after spin_limit polls.
int tree_sample_parts();
int tree_sample_default_spin_limit();
size_t tree_sample_group_bytes();
hipError_t tree_sample_max_groups(int dtype, int* out_groups);
bool tree_sample_fits(int vocab, int dtype);
hipError_t launch_tree_sample(int batch, int max_nodes, int vocab, int dtype, bool vec,
                              const int32_t* parent, const int32_t* token, const int32_t* n_nodes,
                              const void* draft, const void* target, const float* temperature,
                              uint64_t seed, uint64_t offset, int32_t* out_length,
                              int32_t* out_path, int32_t* out_extra, uint64_t* shares,
                              uint64_t* ctl, int spin_limit, int n_groups, hipStream_t stream);

// Scalar-only accept on gathered log-probability pairs.
hipError_t launch_accept_scalar(int batch, int gamma, const float* logprobs, uint64_t seed,
                                uint64_t offset, int32_t* out_len, hipStream_t stream);

// Raw Philox words of every (b, i) block, for tests.
hipError_t launch_philox_words(int batch, int gamma, uint64_t seed, uint64_t offset,
                               uint32_t* out, hipStream_t stream);

}  // namespace specv
