// Residual / bonus kernels: draw the extra token of every sampled sequence.
//
// At the first rejected position k < G the token comes from the residual
// r_v = max(0, p_k(v) - q_k(v)); when all G drafts were kept it is the bonus
// token, r_v = p_G(v) (Speculative Speculative Decoding summary, section 2,
// Saguaro challenge 2: the residual distribution is what the bonus token is
// sampled from). The draw inverts u_res * S on the prefix sums of r in
// vocabulary order: the token is the first v whose inclusive prefix exceeds
// u_res * S, S = sum_v r_v.
//
// Work layout. The vocabulary of a row is cut into tiles of 64 groups (a group
// is one 16-byte load: 8 bf16 or 4 fp32 logits; one logit on the element path).
//   residual_tiles: grid = B * nsplit workgroups of four wavefronts; each
//     wavefront streams whole tiles (lane l reads group 64*t + l of both rows,
//     so one load instruction covers 1 KiB of consecutive memory), and stores
//     one fp32 sum per tile: the groups' pairwise fp32 sums reduced by a fixed
//     DPP butterfly across the wavefront.
//   residual_locate: one wavefront per sequence prefix-sums the tile sums in
//     fp64, finds the tile holding u_res * S, recomputes that tile's group sums
//     with the same arithmetic, scans them in fp64 to find the group and walks
//     the group's elements to find the token.
// The kernel boundary makes the tile sums visible to every XCD; all sums have
// a fixed order, so the result is bitwise reproducible.
//
// p and q are recomputed from the row normalisers (m, s) of the row kernel,
// p_v = 2^(fma(x_v, log2e, -m_p)) / s_p and the same for q, i.e. under the
// normalisers the accept test used. The kernels work with the residual scaled
// by the constant s_q, r'_v = max(0, fma(p'_v, s_q / s_p, -q'_v)) with
// p' = 2^(fma(x, log2e, -m)), which the inversion does not see (u * S scales
// with it) and which costs one fused multiply-add per logit pair. The bonus
// row uses p' itself.
#include "accept.hpp"

namespace specv {
namespace {

constexpr int kTile = 64;  // groups per tile = lanes per wavefront
constexpr int kResidualFusedMaxTiles = 16384;  // LDS tile sums of the fused kernel (64 KiB)
constexpr size_t kTreeLdsBytes = 16384;       // LDS tile sums of one part of a tree (4096 tiles)

// The one or two rows of a sequence at its first rejection.
struct SeqRows {
    const void* prow;
    const void* qrow;
    bool p_only;  // bonus row (or the empty-residual fallback): r' = p'
    float inv_t;
    float mp, mq;   // base-2 references of the rows
    float ratio;    // s_q / s_p
};

// Row pointers of sequence b at position k (needs only the accept outcome).
template <int DT>
__device__ inline void seq_row_ptrs(SeqRows& s, const void* draft, const void* target, int G,
                                    int vocab, int b, int k) {
    s.p_only = k == G;
    s.prow = row_ptr(target, DT, static_cast<size_t>(b) * (G + 1) + k, vocab);
    s.qrow = s.p_only ? s.prow : row_ptr(draft, DT, static_cast<size_t>(b) * G + k, vocab);
}

// Scaling coefficients of those rows, as the accept kernel left them.
__device__ inline void seq_row_coefs(SeqRows& s, const SeqState& st) {
    s.inv_t = st.inv_t;
    s.mp = st.mp;
    s.mq = st.mq;
    s.ratio = st.ratio;
}

template <int DT, bool VEC, bool NT>
struct GroupIO {
    using Ld = Loader<DT, VEC>;
    static constexpr int W = Ld::W;
    typename Ld::raw_t p, q;

    // Both rows are always loaded (for a bonus row qrow == prow), so a batch
    // of loads has no branches and the compiler can wait for each group's
    // loads alone instead of for everything in flight.
    __device__ inline void load(const SeqRows& s, int g) {
        p = Ld::template load_as<NT>(s.prow, g);
        q = Ld::template load_as<NT>(s.qrow, g);
    }

    // r' of the group's elements, in index order.
    __device__ inline void residual(const SeqRows& s, float (&r)[W]) const {
        float zp[W];
        Ld::unpack(p, zp);
        if (s.p_only) {
#pragma unroll
            for (int e = 0; e < W; ++e)
                r[e] = fast_exp2(__builtin_fmaf(scale_logit(zp[e], s.inv_t), kLog2e, -s.mp));
            return;
        }
        float zq[W];
        Ld::unpack(q, zq);
#pragma unroll
        for (int e = 0; e < W; ++e) {
            const float pv = fast_exp2(__builtin_fmaf(scale_logit(zp[e], s.inv_t), kLog2e, -s.mp));
            const float qv = fast_exp2(__builtin_fmaf(scale_logit(zq[e], s.inv_t), kLog2e, -s.mq));
            r[e] = fmaxf(__builtin_fmaf(pv, s.ratio, -qv), 0.0f);
        }
    }
};

template <int N>
__device__ inline float pairwise(const float (&r)[N]) {
    float t[N];
#pragma unroll
    for (int e = 0; e < N; ++e)
        t[e] = r[e];
#pragma unroll
    for (int w = 1; w < N; w <<= 1) {
#pragma unroll
        for (int i = 0; i + w < N; i += 2 * w)
            t[i] += t[i + w];
    }
    return t[0];
}

// Tile sum of the 64 lanes' group sums, in a fixed order: DPP butterfly
// within each row of 16 lanes, then the row broadcasts, then lane 63 holds the
// total, which is returned to every lane.
template <int CTRL, int ROW_MASK>
__device__ inline float add_dpp(float v) {
    const int t = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false);
    return v + __int_as_float(t);
}

__device__ inline float tile_reduce(float v) {
    v = add_dpp<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v = add_dpp<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v = add_dpp<0x141, 0xF>(v);  // row_half_mirror
    v = add_dpp<0x140, 0xF>(v);  // row_mirror: every lane holds its row's sum
    v = add_dpp<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v = add_dpp<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3: lane 63 = total
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// With ACC the kernel also runs the accept step (small batches, where the
// separate accept launch would be a large part of the call): wavefront 0 of
// every split decides its sequence, split 0 alone writes the accept outputs,
// and the state reaches the other wavefronts through LDS.
template <int DT, bool VEC, int U, bool NT, bool ACC>
__global__ __launch_bounds__(kBlock) void residual_tiles_kernel(
    const void* __restrict__ draft, const void* __restrict__ target, int gamma, int vocab,
    int ntiles, int tiles_per_split, int tiles_per_row, const SeqState* __restrict__ seq,
    float* __restrict__ tile_sums, AcceptArgs acc) {
    using IO = GroupIO<DT, VEC, NT>;
    constexpr int W = IO::W;
    // grid: x = sequence, y = vocabulary split
    const int b = blockIdx.x;
    const int wid = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int lane = threadIdx.x & 63;
    SeqState st;
    if constexpr (ACC) {
        __shared__ SeqState acc_state;
        if (wid == 0) {
            const SeqState s0 = accept_sequence(acc, b, blockIdx.y == 0);
            if (lane == 0)
                acc_state = s0;
        }
        __syncthreads();
        st = acc_state;
    } else {
        (void)acc;
        st = seq[b];
    }
    if (st.mode != 1)
        return;  // greedy or rejected sequence: nothing to draw
    const int groups = vocab / W;
    const int t0 = blockIdx.y * tiles_per_split;
    const int t1 = t0 + tiles_per_split < ntiles ? t0 + tiles_per_split : ntiles;
    float* out = tile_sums + static_cast<size_t>(b) * tiles_per_row;

    // Double-buffered: the loads of the next batch are in flight while this
    // batch is reduced.
    SeqRows s;
    seq_row_ptrs<DT>(s, draft, target, gamma, vocab, b, st.k);
    // Loads are unconditional: a group past the split or the row reads group 0
    // of the row instead (always in bounds) and is not used.
    auto load_batch = [&](IO (&io)[U], int t) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int g = (t + u * kWaves) * kTile + lane;
            const bool used = t + u * kWaves < t1 && g < groups;
            io[u].load(s, used ? g : 0);
        }
    };
    auto reduce_batch = [&](const IO (&io)[U], int t) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tt = t + u * kWaves;
            if (tt >= t1)
                break;  // wave-uniform
            const int g = tt * kTile + lane;
            float gs = 0.0f;
            if (g < groups) {
                float r[W];
                io[u].residual(s, r);
                gs = pairwise(r);
            }
            const float ts = tile_reduce(gs);
            if (lane == 0)
                out[tt] = ts;
        }
    };
    constexpr int kStep = kWaves * U;
    IO buf_a[U], buf_b[U];
    int t = t0 + wid;
    load_batch(buf_a, t);
    seq_row_coefs(s, st);
    // The next batch is loaded unconditionally (a batch past the split reads
    // group 0, which is in cache, and is never reduced): with no branch around
    // the loads, and no loop exit between the two halves, the compiler waits
    // for exactly the batch being reduced.
    const int nb = t < t1 ? (t1 - t + kStep - 1) / kStep : 0;
    for (int i = 0; i + 2 <= nb; i += 2) {
        load_batch(buf_b, t + kStep);
        reduce_batch(buf_a, t);
        load_batch(buf_a, t + 2 * kStep);
        reduce_batch(buf_b, t + kStep);
        t += 2 * kStep;
    }
    if (nb & 1)
        reduce_batch(buf_a, t);
}

// 64-bit DPP move: both halves take the same lane pattern; lanes whose source
// lies outside the row, or whose row is not in ROW_MASK, read +0.0.
template <int CTRL, int ROW_MASK>
__device__ inline double dpp_f64(double v) {
    const unsigned long long u = static_cast<unsigned long long>(__double_as_longlong(v));
    const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(u & 0xffffffffu), CTRL, ROW_MASK,
                                               0xF, true);
    const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(u >> 32), CTRL, ROW_MASK, 0xF,
                                               true);
    return __longlong_as_double(static_cast<long long>(
        (static_cast<unsigned long long>(static_cast<unsigned>(hi)) << 32) | static_cast<unsigned>(lo)));
}

// Inclusive prefix over the 64 lanes in fp64 (lane order), in a fixed order:
// shifts by 1, 2, 4 and 8 within each row of 16 lanes, then the row totals
// are carried forward by the row broadcasts.
__device__ inline double wave_inclusive_scan(double v) {
    v += dpp_f64<0x111, 0xF>(v);  // row_shr:1
    v += dpp_f64<0x112, 0xF>(v);  // row_shr:2
    v += dpp_f64<0x114, 0xF>(v);  // row_shr:4
    v += dpp_f64<0x118, 0xF>(v);  // row_shr:8
    v += dpp_f64<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_f64<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

// Lane `lane`'s value (a wave-uniform lane index) to every lane, without a
// round trip through LDS.
__device__ inline double readlane_f64(double v, int lane) {
    const unsigned long long u = static_cast<unsigned long long>(__double_as_longlong(v));
    const unsigned lo = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(u & 0xffffffffu), lane));
    const unsigned hi = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(u >> 32), lane));
    return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo));
}

__device__ inline double lane63_f64(double v) { return readlane_f64(v, 63); }

__device__ inline int first_lane(bool flag) {
    const unsigned long long m = __ballot(flag);
    return m ? __ffsll(static_cast<long long>(m)) - 1 : 64;
}

__device__ inline int wave_max_int(int v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const int o = __shfl_xor(v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

// The tile sums `ts` (fp32) of one row, cut into 64 contiguous runs: lane l
// sums run l in fp64 and the wavefront scans the runs; the last lane's prefix
// is the row total S.
// With REGS, runs of up to kRunRegs tiles (rows of up to 64 * kRunRegs tiles)
// are read into registers with reads issued together (clamped into range, the
// values past the run masked to zero) and walked again from there by
// locate_tile; otherwise, and for longer runs, they are read in a loop. Both
// forms add in the same order. The verifier's draw takes REGS (its 1.2 us of
// dependent LDS reads drop to one round trip); the tree sampler, whose walk
// holds more registers, the loop.
constexpr int kRunRegs = 8;

struct TileRuns {
    int a0, a1;       // this lane's run [a0, a1)
    int last_pos;     // its last tile with mass, or -1
    bool in_regs;     // the run's values are in v (wave-uniform)
    double mine;      // its run's sum
    double inc;       // inclusive prefix of the runs through this lane
    float v[kRunRegs];
};

template <bool REGS>
__device__ inline TileRuns tile_runs(const float* ts, int ntiles) {
    const int lane = threadIdx.x & 63;
    const int per = (ntiles + 63) / 64;
    TileRuns tr;
    tr.a0 = lane * per < ntiles ? lane * per : ntiles;
    tr.a1 = tr.a0 + per < ntiles ? tr.a0 + per : ntiles;
    tr.mine = 0.0;
    tr.last_pos = -1;
    tr.in_regs = REGS && ntiles >= 1 && per <= kRunRegs;
    if (REGS && tr.in_regs) {
#pragma unroll
        for (int j = 0; j < kRunRegs; ++j) {
            const int t = tr.a0 + j < ntiles ? tr.a0 + j : ntiles - 1;
            const float v = ts[t];
            tr.v[j] = tr.a0 + j < tr.a1 ? v : 0.0f;
        }
        // Straight-line code: the values past the run are +0, which adds
        // nothing to a non-negative sum and never holds mass.
#pragma unroll
        for (int j = 0; j < kRunRegs; ++j) {
            tr.mine += static_cast<double>(tr.v[j]);
            tr.last_pos = tr.v[j] > 0.0f ? tr.a0 + j : tr.last_pos;
        }
    } else {
        for (int t = tr.a0; t < tr.a1; ++t) {
            const float v = ts[t];
            tr.mine += static_cast<double>(v);
            if (v > 0.0f)
                tr.last_pos = t;
        }
    }
    tr.inc = wave_inclusive_scan(tr.mine);
    return tr;
}

// Locate the tile holding tau: the lane whose run crosses tau walks it.
// Returns the tile and writes the fp64 prefix before it; when tau lies beyond
// the total (rounding only), returns the last tile with mass and writes -1
// (take its last positive element).
template <bool REGS>
__device__ inline int locate_tile(const float* ts, const TileRuns& tr, double tau, double* P_out) {
    int hit = -1;
    double before = 0.0;
    double acc = tr.inc - tr.mine;
    if (REGS && tr.in_regs) {
        // Straight-line code: the +0 values past the run never hit, and the
        // running sum is unused once the hit is found.
#pragma unroll
        for (int j = 0; j < kRunRegs; ++j) {
            const float v = tr.v[j];
            const double next = acc + static_cast<double>(v);
            const bool h = hit < 0 && v > 0.0f && next > tau;
            before = h ? acc : before;
            hit = h ? tr.a0 + j : hit;
            acc = next;
        }
    } else {
        for (int t = tr.a0; t < tr.a1 && hit < 0; ++t) {
            const float v = ts[t];
            const double next = acc + static_cast<double>(v);
            if (v > 0.0f && next > tau) {
                hit = t;
                before = acc;
            }
            acc = next;
        }
    }
    const int fl = first_lane(hit >= 0);
    if (fl < 64) {
        *P_out = readlane_f64(before, fl);
        return __builtin_amdgcn_readlane(hit, fl);
    }
    *P_out = -1.0;
    return wave_max_int(tr.last_pos);
}

// Highest lane whose flag is set, or -1.
__device__ inline int last_lane(bool flag) {
    const unsigned long long m = __ballot(flag);
    return m ? 63 - __clzll(static_cast<long long>(m)) : -1;
}

// The group and element levels of the draw inside one tile. Lane l holds the
// sum gs of group 64*tile + l (0 past the row), formed as the tile sums were;
// P is the fp64 prefix before the tile (P < 0: take the tile's last positive
// element). The group is the first whose fp64 running sum passes tau; its W
// elements are then reloaded, one per lane, their residuals formed with the
// streaming arithmetic, scanned in fp64 from the prefix before the group, and
// the first element that carries the sum past tau is the token. When rounding
// leaves the walk short of tau, the chosen group's last positive element is
// taken. Every lane returns the token.
template <int DT, bool VEC>
__device__ inline int locate_in_tile(const SeqRows& s, int tile, float gs, double P, double tau) {
    constexpr int W = Group<DT, VEC>::W;
    const int lane = threadIdx.x & 63;
    const double inc = wave_inclusive_scan(static_cast<double>(gs));
    bool take_last = P < 0.0;
    int gl = take_last ? 64 : first_lane(gs > 0.0f && P + inc > tau);
    double Pg = 0.0;
    if (gl < 64) {
        Pg = P + readlane_f64(inc - static_cast<double>(gs), gl);
    } else {
        gl = last_lane(gs > 0.0f);
        take_last = true;
        if (gl < 0)
            gl = 0;  // unreachable: a tile with mass has a group with mass
    }
    const long g = static_cast<long>(tile) * kTile + gl;
    float r = 0.0f;
    if (lane < W) {
        // Both logits are loaded before either is used (for a bonus row qrow
        // is prow), and the result is selected, so the two loads share one
        // memory round trip instead of the second waiting behind the first
        // (the empty asm keeps the scheduler from placing a use between them).
        const long v = g * W + lane;
        const uint32_t bp = load_logit_bits(s.prow, DT, v);
        const uint32_t bq = load_logit_bits(s.qrow, DT, v);
        asm volatile("" ::"v"(bp), "v"(bq));  // neither is used before both are issued
        const float zp = logit_of_bits(bp, DT);
        const float zq = logit_of_bits(bq, DT);
        const float pv = fast_exp2(__builtin_fmaf(scale_logit(zp, s.inv_t), kLog2e, -s.mp));
        const float qv = fast_exp2(__builtin_fmaf(scale_logit(zq, s.inv_t), kLog2e, -s.mq));
        const float rr = fmaxf(__builtin_fmaf(pv, s.ratio, -qv), 0.0f);
        r = s.p_only ? pv : rr;
    }
    const double einc = wave_inclusive_scan(static_cast<double>(r));
    int e = take_last ? 64 : first_lane(r > 0.0f && Pg + einc > tau);
    if (e >= 64) {
        e = last_lane(r > 0.0f);
        if (e < 0)
            e = W - 1;  // unreachable: a group with mass has an element with mass
    }
    return static_cast<int>(g * W + e);
}

// The sum of group 64*tile + l of the row pair (lane l), recomputed with the
// streaming arithmetic (0 past the row).
template <int DT, bool VEC, bool NT>
__device__ inline float group_sum_of(const SeqRows& s, int tile, int groups) {
    using IO = GroupIO<DT, VEC, NT>;
    constexpr int W = IO::W;
    const int g = tile * kTile + (threadIdx.x & 63);
    float gs = 0.0f;
    if (g < groups) {
        IO io;
        io.load(s, g);
        float r[W];
        io.residual(s, r);
        gs = pairwise(r);
    }
    return gs;
}

// Token inside one tile, from its group sums recomputed by re-reading it.
template <int DT, bool VEC, bool NT>
__device__ inline int scan_tile(const SeqRows& s, int tile, int groups, double P, double tau) {
    return locate_in_tile<DT, VEC>(s, tile, group_sum_of<DT, VEC, false>(s, tile, groups), P, tau);
}

template <int DT, bool VEC, bool NT>
__device__ inline double tile_sum_of(const SeqRows& s, int t, int groups) {
    return static_cast<double>(tile_reduce(group_sum_of<DT, VEC, NT>(s, t, groups)));
}

// The draw from the tile sums `ts` (global memory or LDS) of one row pair, by
// one wavefront, with uniform u: total S, the tile holding tau = u * S, then
// the token inside it; the empty-residual fallback streams p at the same
// position. Every lane returns the token.
template <int DT, bool VEC, bool NT>
__device__ inline int draw_p_fallback(SeqRows& s, float u, int ntiles, int groups);

// The token at position tau of the weights whose tile sums are ts.
template <int DT, bool VEC, bool NT>
__device__ inline int draw_at(const SeqRows& s, double tau, const float* ts, int ntiles, int groups) {
    const TileRuns tr = tile_runs<false>(ts, ntiles);
    double P;
    const int tile = locate_tile<false>(ts, tr, tau, &P);
    return scan_tile<DT, VEC, NT>(s, tile, groups, P, tau);
}

template <int DT, bool VEC, bool NT>
__device__ inline int draw_token(SeqRows& s, float u, const float* ts, int ntiles, int groups) {
    const TileRuns tr = tile_runs<true>(ts, ntiles);
    const double S = lane63_f64(tr.inc);
    if (S > 0.0) {
        const double tau = static_cast<double>(u) * S;
        double P;
        const int tile = locate_tile<true>(ts, tr, tau, &P);
        return scan_tile<DT, VEC, NT>(s, tile, groups, P, tau);
    }
    return draw_p_fallback<DT, VEC, NT>(s, u, ntiles, groups);
}

// The draw with every group sum of the row kept (gs_lds[64 * tile + l]):
// the tile's group sums are read instead of recomputed.
template <int DT, bool VEC, bool NT>
__device__ inline int draw_token_gs(SeqRows& s, float u, const float* ts, const float* gs_lds,
                                    int ntiles, int groups) {
    const TileRuns tr = tile_runs<true>(ts, ntiles);
    const double S = lane63_f64(tr.inc);
    if (S > 0.0) {
        const double tau = static_cast<double>(u) * S;
        double P;
        const int tile = locate_tile<true>(ts, tr, tau, &P);
        const float gs = gs_lds[tile * kTile + (threadIdx.x & 63)];
        return locate_in_tile<DT, VEC>(s, tile, gs, P, tau);
    }
    return draw_p_fallback<DT, VEC, NT>(s, u, ntiles, groups);
}

// Empty residual (possible only through rounding when p and q agree to within
// fp32): draw from p at the same position instead. Slow path: the wavefront
// streams the row twice.
template <int DT, bool VEC, bool NT>
__device__ inline int draw_p_fallback(SeqRows& s, float u, int ntiles, int groups) {
    s.p_only = true;
    double sp = 0.0;
    for (int t = 0; t < ntiles; ++t)
        sp += tile_sum_of<DT, VEC, NT>(s, t, groups);
    const double tau = static_cast<double>(u) * sp;
    double P = 0.0;
    int tile = -1;
    for (int t = 0; t < ntiles && tile < 0; ++t) {
        const double tsum = tile_sum_of<DT, VEC, NT>(s, t, groups);
        if (tsum > 0.0 && P + tsum > tau)
            tile = t;
        else
            P += tsum;
    }
    if (tile < 0) {
        tile = ntiles - 1;
        P = -1.0;
    }
    return scan_tile<DT, VEC, NT>(s, tile, groups, P, tau);
}

// The draw of one sequence (one wavefront), written to its extra token.
template <int DT, bool VEC, bool NT>
__device__ inline void locate_emit(SeqRows& s, const SeqState& st, const float* ts, int ntiles,
                                   int groups, int G, int b, int32_t* out_tok) {
    const int token = draw_token<DT, VEC, NT>(s, st.u_res, ts, ntiles, groups);
    if ((threadIdx.x & 63) == 0)
        out_tok[static_cast<size_t>(b) * (G + 1) + st.k] = token;
}

template <int DT, bool VEC, bool NT>
__global__ __launch_bounds__(64) void residual_locate_kernel(
    const void* __restrict__ draft, const void* __restrict__ target, int gamma, int vocab,
    int ntiles, int tiles_per_row, const SeqState* __restrict__ seq,
    const float* __restrict__ tile_sums, int32_t* __restrict__ out_tok) {
    constexpr int W = Group<DT, VEC>::W;
    const int b = blockIdx.x;
    const SeqState st = seq[b];
    if (st.mode != 1)
        return;
    SeqRows s;
    seq_row_ptrs<DT>(s, draft, target, gamma, vocab, b, st.k);
    seq_row_coefs(s, st);
    locate_emit<DT, VEC, NT>(s, st, tile_sums + static_cast<size_t>(b) * tiles_per_row, ntiles,
                             vocab / W, gamma, b, out_tok);
}

// One workgroup of 12 wavefronts per sequence: the wavefronts stream the
// sequence's tiles with the tile kernel's arithmetic and per-tile sums, keep
// the tile sums in LDS (with GS also every group sum, so the draw reads the
// chosen tile's group sums instead of recomputing them), and after one
// barrier wavefront 0 draws the token.
// Used when there are enough sequences to give every CU a workgroup; it saves
// the second launch and the round trip of the tile sums through memory.
// Tiles are handed out by an LDS counter (each wavefront holds two in flight
// and asks for the next one a tile ahead), so wavefronts whose loads return
// late take fewer tiles and all reach the barrier together.
// Twelve wavefronts (three per SIMD) measured about 1 % faster than sixteen
// and clearly faster than ten or eight: fewer tiles in flight per CU shorten
// the spread of the workgroups' stream ends, down to where the arithmetic
// between loads is no longer hidden.
constexpr int kFusedBlock = 768;

template <int DT, bool VEC, bool NT, int BLOCK, bool GS>
__global__ __launch_bounds__(BLOCK) void residual_fused_kernel(
    const void* __restrict__ draft, const void* __restrict__ target, int gamma, int vocab,
    int ntiles, const SeqState* __restrict__ seq, int32_t* __restrict__ out_tok) {
    using IO = GroupIO<DT, VEC, NT>;
    constexpr int W = IO::W;
    constexpr int kFusedWaves = BLOCK / 64;
    extern __shared__ float lds_ts[];  // [ntiles] tile sums, then with GS [64 * ntiles] group sums
    float* const lds_gs = lds_ts + ntiles;
    __shared__ int next_tile;
    const int b = blockIdx.x;
    const SeqState st = seq[b];
    // The arguments and the whole state are asked for here, before the first
    // branch: left to itself the compiler reads the rest of the state and
    // the other arguments after the mode test, and the draft row's base
    // after the barrier, each a further scalar round trip before the first
    // tile's loads can leave.
    asm volatile("" ::"s"(draft), "s"(target), "s"(gamma), "s"(vocab), "s"(ntiles), "s"(out_tok));
    asm volatile("" ::"s"(st.k), "s"(st.u_res), "s"(st.inv_t), "s"(st.mp), "s"(st.mq), "s"(st.ratio));
    if (st.mode != 1)
        return;  // greedy or rejected sequence: nothing to draw
    const int groups = vocab / W;
    const int wid = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int lane = threadIdx.x & 63;
    SeqRows s;
    seq_row_ptrs<DT>(s, draft, target, gamma, vocab, b, st.k);
    // Loads are unconditional: a tile past the row reads group 0 instead and
    // is not reduced.
    auto load_tile = [&](IO& io, int t) {
        const int g = t * kTile + lane;
        io.load(s, t < ntiles && g < groups ? g : 0);
    };
    IO buf_a, buf_b;
    int ta = wid, tb = wid + kFusedWaves;
    // The first tile leaves before the barrier, which guards only the
    // counter.
    load_tile(buf_a, ta);
    if (threadIdx.x == 0)
        next_tile = 2 * kFusedWaves;  // tiles below are dealt out statically
    __syncthreads();
    auto reduce_tile = [&](const IO& io, int t) {
        if (t >= ntiles)
            return;  // wave-uniform
        const int g = t * kTile + lane;
        float gs = 0.0f;
        if (g < groups) {
            float r[W];
            io.residual(s, r);
            gs = pairwise(r);
        }
        if constexpr (GS)
            lds_gs[g] = gs;
        const float ts = tile_reduce(gs);
        if (lane == 0)
            lds_ts[t] = ts;
    };
    // The counter's answer stays in lane 0's register until the tile after
    // next is loaded, so the LDS atomic completes behind a tile's arithmetic.
    auto grab = [&]() {
        int v = 0;
        if (lane == 0)
            v = atomicAdd(&next_tile, 1);
        return v;
    };
    auto uniform = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
    seq_row_coefs(s, st);
    int tn = grab();
    // Counter values only grow, so once ta is past the row so is every later
    // tile, and the single exit at the head leaves nothing in flight unused.
    while (ta < ntiles) {
        load_tile(buf_b, tb);
        reduce_tile(buf_a, ta);
        ta = uniform(tn);
        tn = grab();
        load_tile(buf_a, ta);
        reduce_tile(buf_b, tb);
        tb = uniform(tn);
        tn = grab();
    }
    __syncthreads();
    if (wid != 0)
        return;
    if constexpr (GS) {
        const int token = draw_token_gs<DT, VEC, NT>(s, st.u_res, lds_ts, lds_gs, ntiles, groups);
        if (lane == 0)
            out_tok[static_cast<size_t>(b) * (gamma + 1) + st.k] = token;
    } else {
        locate_emit<DT, VEC, NT>(s, st, lds_ts, ntiles, groups, gamma, b, out_tok);
    }
}

// ----------------------------------------------- sampled draft trees ---
//
// Multi-step speculative sampling over a draft tree (SpecInfer, ASPLOS 2024,
// stochastic tree verification, with one draft distribution per node): one
// 1024-thread workgroup per tree walks it from the root. At node u the target
// is pi = (p_u - c q_u)^+ / Z: c = 0, Z = 1 on arrival, and after a rejection
// c <- c + Z, Z <- sum_v (p_u - c q_u)^+, which is norm(max(0, pi - q_u))
// written in closed form. Each step that needs a whole row is one pass of the
// workgroup over it:
//   * arrival at u: (m, s) of target row u, and of draft row u before its
//     first child is tried (the row kernel's online base-2 form);
//   * a rejection: the tile sums of r' = max(0, fma(p', s_q / (c s_p), -q'))
//     (the residual draw's arithmetic, r' = (s_q / c) (p - c q)^+), whose total
//     gives Z;
//   * the end: the same tile sums (p' alone when c = 0) and the residual
//     draw's inversion with the uniform of block (L, b), word 1.
// The accept test of child s is the verifier's, in fp64: log u < log pi(t) -
// log q(t) with u from block (s - 1, b), word 0, and log pi(t) = x_p(t) -
// lse_p while c = 0. At T = 0 the walk follows the raw-logit argmax instead.
// ---------------------------------------------------------------------------
// Sampled verification of draft trees (multi-step speculative sampling with
// one draft distribution per node). The walk through one tree is sequential,
// and one CU streams a row pair with exp2 on every logit at far below its
// share of HBM, so a lone long walk would set the time of the whole call.
// Each tree is therefore split over kTreeParts workgroups that each own a
// contiguous run of whole tiles of the vocabulary. Every part runs the same
// walk: after each pass it publishes its share (row maxima and sums, the
// residual total, the argmax) and reads the other parts' shares; all parts
// merge them in one fixed order, so they take identical decisions. The part
// whose run holds the final draw position writes the extra token.
//
// Exchange: a share travels as 16-bit pieces, each in a 64-bit word whose
// upper 48 bits carry the pass's tag, (call << 20) | pass. A part writes its
// pieces with device-coherent 64-bit stores and polls its partners' pieces
// with device-coherent loads until every tag matches, so one round trip both
// signals and delivers. Pieces live in two slots by pass parity (a part
// cannot run two passes ahead of a partner, so the slot it reads holds either
// the partner's share of this pass or an older one). The call number is read
// from a device word at the start of the launch and advanced by the last
// workgroup to finish it, so every launch (each replay of a captured graph
// included) tags its exchanges anew; a tag from an earlier launch can only
// match after 2^28 launches that left the slot untouched. Release and acquire
// fences are not used: at device scope they write back and invalidate the
// whole L2 of an XCD, which a thousand workgroups exchanging at once
// serialise. The grid never exceeds what the device holds at once, so every
// part becomes resident; every wait is still bounded: a partner missing for
// the spin limit (kTreeSpinLimit polls unless the context sets another) makes
// the part give up, and all parts finish.
//
// Outputs: part 0 writes the whole outcome of a tree (the drawing part hands
// it the token through one more exchange), so a tree is reported by the one
// part that saw every exchange of it: its outcome, -1 for invalid input, or
// -2 when part 0 or a partner gave up waiting (counted in the control block).
constexpr int kTreeParts = 4;
constexpr int kTreeBlock = 256;
constexpr int kTreeWaves = kTreeBlock / 64;
constexpr int kTreeSpinLimit = 1 << 20;

// One part's share of a pass, six 32-bit words: a norm pass puts the target
// row's base-2 maximum in word 0 and its sum (fp64) in words 2-3, the draft
// row's in word 1 and words 4-5; a tile pass its residual total (fp64) in
// words 2-3; an argmax pass the best raw logit in word 0 and its token in 1.
struct TreePart {
    uint32_t w[6];
};
constexpr int kShareHalves = 12;  // 16-bit pieces of a share

__device__ inline void part_set_f(TreePart& p, int i, float x) { p.w[i] = __float_as_uint(x); }
__device__ inline void part_set_d(TreePart& p, int i, double x) {
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(x));
    p.w[i] = static_cast<uint32_t>(b);
    p.w[i + 1] = static_cast<uint32_t>(b >> 32);
}
__device__ inline float part_f(const TreePart& p, int i) { return __uint_as_float(p.w[i]); }
__device__ inline double part_d(const TreePart& p, int i) {
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(p.w[i + 1]) << 32) | p.w[i]));
}
__device__ inline TreePart part_zero() {
    TreePart p;
#pragma unroll
    for (int i = 0; i < 6; ++i)
        p.w[i] = 0;
    return p;
}

struct TreeSampleArgs {
    const int32_t* parent;
    const int32_t* token;
    const int32_t* n_nodes;
    const void* draft;
    const void* target;
    const float* temperature;
    int B, M, V;
    uint64_t seed, offset;
    int32_t* out_length;
    int32_t* out_path;
    int32_t* out_extra;
    uint64_t* shares;  // [groups][2][kTreeParts][kShareHalves] tagged pieces
    uint64_t* ctl;     // [0] launches finished, [1] workgroups finished in this
                       // launch, [2] trees given up (cumulative)
    int spin_limit;    // polls before a part gives up on a partner
};

struct TreeShared {
    int parent[256];
    int token[256];
    int path[256];
    float red_f[kTreeWaves];
    double red_d[kTreeWaves];
    int red_i[kTreeWaves];
    TreePart xp[kTreeParts];
    double tot_keep[kTreeParts];  // per-part residual totals of the draw's tile sums
    uint64_t nodes[kTreeBlock / 64];  // a set of nodes, one bit each (node_set)
    int flag;
    int decision;
    int ok;
};

// The set of nodes i < n (one per thread, M <= kTreeBlock) with pred(i)
// true, into sh.nodes; every thread then reads it. Two barriers.
template <class P>
__device__ inline void node_set(TreeShared& sh, int n, P&& pred) {
    const int i = threadIdx.x;
    const uint64_t m = __ballot(i < n && pred(i));
    __syncthreads();  // earlier readers of sh.nodes are done
    if ((i & 63) == 0)
        sh.nodes[i >> 6] = m;
    __syncthreads();
}

// The lowest node >= s in sh.nodes, or `none`.
__device__ inline int node_set_next(const TreeShared& sh, int s, int none) {
    for (int w = s >> 6; w < kTreeBlock / 64; ++w) {
        uint64_t m = sh.nodes[w];
        if (w == (s >> 6))
            m &= ~0ULL << (s & 63);
        if (m)
            return w * 64 + __ffsll(static_cast<long long>(m)) - 1;
    }
    return none;
}

// Largest value over the wavefront's lanes, returned to every lane: the
// inclusive scan's pattern (shifts by 1, 2, 4 and 8 within each row of 16
// lanes, then the row broadcasts) leaves it in lane 63. A lane whose source
// is out of range keeps its own value.
template <int CTRL, int ROW_MASK>
__device__ inline float max_dpp(float v) {
    const int t = __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROW_MASK,
                                              0xF, false);
    return fmaxf(v, __int_as_float(t));
}

__device__ inline float wave_max_f32(float v) {
    v = max_dpp<0x111, 0xF>(v);  // row_shr:1
    v = max_dpp<0x112, 0xF>(v);  // row_shr:2
    v = max_dpp<0x114, 0xF>(v);  // row_shr:4
    v = max_dpp<0x118, 0xF>(v);  // row_shr:8
    v = max_dpp<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v = max_dpp<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Block-wide sum of the tree workgroup in a fixed order (every thread gets
// it): the lanes by the DPP scan, then the wavefronts in order.
__device__ inline double tree_block_sum(double v, TreeShared& sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    v = lane63_f64(wave_inclusive_scan(v));
    __syncthreads();
    if (lane == 0)
        sh.red_d[w] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < kTreeWaves; ++i)
        t += sh.red_d[i];
    return t;
}

// Largest raw logit, lowest index on ties (index 0x7fffffff when empty).
__device__ inline void tree_block_argmax(float v, int i, TreeShared& sh, float* bv_out,
                                         int* bi_out) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(v, off, 64);
        const int oi = __shfl_xor(i, off, 64);
        if (ov > v || (ov == v && oi < i)) {
            v = ov;
            i = oi;
        }
    }
    __syncthreads();
    if (lane == 0) {
        sh.red_f[w] = v;
        sh.red_i[w] = i;
    }
    __syncthreads();
    float bv = sh.red_f[0];
    int bi = sh.red_i[0];
    for (int k = 1; k < kTreeWaves; ++k) {
        if (sh.red_f[k] > bv || (sh.red_f[k] == bv && sh.red_i[k] < bi)) {
            bv = sh.red_f[k];
            bi = sh.red_i[k];
        }
    }
    *bv_out = bv;
    *bi_out = bi;
}

// One pass over R rows at once: 64-group tiles w, w + kTreeWaves, ... per
// wavefront, D tiles of every row in flight in a register ring (loads past the
// end are clamped onto group 0 and never used). f(group index, in range,
// values of each row) is called by whole wavefronts; lanes past the last
// group get in range = false (their values are group 0's). groups >= 1.
template <int DT, bool VEC, bool NT, int R, int D, class F>
__device__ inline void tree_stream(const void* const (&rows)[R], int groups, F&& f) {
    using Ld = Loader<DT, VEC>;
    using raw_t = typename Ld::raw_t;
    constexpr int W = Ld::W;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int ntiles = (groups + kTile - 1) / kTile;
    auto addr = [&](int k) {
        const int g = (wid + k * kTreeWaves) * kTile + lane;
        return g < groups ? g : 0;
    };
    raw_t buf[D][R];
    // Issue the first loads in slot order (the waits below count loads in
    // flight, so a reordered prologue would make the first use wait for all).
#pragma unroll
    for (int j = 0; j < D; ++j) {
#pragma unroll
        for (int r = 0; r < R; ++r)
            buf[j][r] = Ld::template load_as<NT>(rows[r], addr(j));
        __builtin_amdgcn_sched_barrier(0);
    }
    const int nb = wid < ntiles ? (ntiles - wid + kTreeWaves - 1) / kTreeWaves : 0;
    for (int k = 0; k < nb; k += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            // Use slot j, then refill it: each slot keeps its registers, so
            // the ring needs no copies (which would wait for every load).
            const int g = (wid + (k + j) * kTreeWaves) * kTile + lane;
            if (k + j < nb) {
                float z[R][W];
#pragma unroll
                for (int r = 0; r < R; ++r)
                    Ld::unpack(buf[j][r], z[r]);
                f(g, g < groups, z);
            }
#pragma unroll
            for (int r = 0; r < R; ++r)
                buf[j][r] = Ld::template load_as<NT>(rows[r], addr(k + j + D));
        }
    }
}

// Online (m, s) of one row in the row kernel's base-2 form: m = fl32(max x *
// log2e), s = sum 2^(fma(x, log2e, -m)).
template <int W>
struct OnlineNorm {
    float m = kNegMax;
    double s = 0.0;

    __device__ inline void add(const float (&z)[W], float inv_t) {
        float x[W];
        float gm = -__builtin_huge_valf();
#pragma unroll
        for (int e = 0; e < W; ++e) {
            x[e] = scale_logit(z[e], inv_t);
            gm = fmaxf(gm, x[e]);
        }
        const float mn = gm * kLog2e;
        if (mn > m) {
            s *= static_cast<double>(fast_exp2(m - mn));
            m = mn;
        }
        float g = 0.0f;
#pragma unroll
        for (int e = 0; e < W; ++e)
            g += fast_exp2(__builtin_fmaf(x[e], kLog2e, -m));
        s += static_cast<double>(g);
    }

    // Merge over the workgroup (every thread gets the part's (m, s)): each
    // wavefront folds its lanes by DPP (the maximum, then the lanes' sums
    // scaled to it), and the wavefronts' pairs are merged in wavefront order
    // through LDS, one exchange for both.
    __device__ inline void finish(TreeShared& sh, float* m_out, double* s_out) const {
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
        const float mw = wave_max_f32(m);
        const double f = m == mw ? 1.0 : static_cast<double>(fast_exp2(m - mw));
        const double sw = lane63_f64(wave_inclusive_scan(s > 0.0 ? s * f : 0.0));
        __syncthreads();  // earlier readers of red_f and red_d are done
        if (lane == 0) {
            sh.red_f[w] = mw;
            sh.red_d[w] = sw;
        }
        __syncthreads();
        float M = sh.red_f[0];
#pragma unroll
        for (int i = 1; i < kTreeWaves; ++i)
            M = fmaxf(M, sh.red_f[i]);
        double S = 0.0;
#pragma unroll
        for (int i = 0; i < kTreeWaves; ++i) {
            const double si = sh.red_d[i];
            const float mi = sh.red_f[i];
            if (si > 0.0)
                S += mi == M ? si : si * static_cast<double>(fast_exp2(mi - M));
        }
        *m_out = M;
        *s_out = S;
    }
};

// (m, s) of the shares in sh.xp, in part order: the target row's, or the
// draft row's when second.
__device__ inline void merge_norm(const TreeShared& sh, bool second, float* m_out, double* s_out) {
    float M = kNegMax;
    for (int j = 0; j < kTreeParts; ++j)
        M = fmaxf(M, part_f(sh.xp[j], second ? 1 : 0));
    double S = 0.0;
    for (int j = 0; j < kTreeParts; ++j) {
        const float mj = part_f(sh.xp[j], second ? 1 : 0);
        const double sj = part_d(sh.xp[j], second ? 4 : 2);
        if (sj > 0.0)
            S += mj == M ? sj : sj * static_cast<double>(fast_exp2(mj - M));
    }
    *m_out = M;
    *s_out = S;
}

constexpr int kTreeDepth1 = 6;  // ring depth of a one-row pass
constexpr int kTreeDepth2 = 3;  // ring depth of a two-row pass

// A part's view of its tree: its run of the vocabulary and the exchange.
struct TreePartView {
    int part;        // 0 .. kTreeParts - 1
    int g0, ng;      // first group and number of groups of the run (ng may be 0)
    int nt;          // tiles of the run
    int W;           // logits per group
    int dt;          // dtype
    uint64_t* shares;  // this group's two slots
    uint64_t tag;      // last published tag
    int spin_limit;    // polls before giving up on a partner
    bool live;       // false once a partner went missing

    __device__ inline const void* sub(const void* row) const {
        const size_t esz = dt == kBF16 ? 2 : 4;
        return static_cast<const char*>(row) + static_cast<size_t>(g0) * W * esz;
    }
};

// Publish this part's share of the next pass and collect all shares into
// sh.xp (part order). Returns false (for every thread) when a partner has not
// published within the spin limit; the view then stops waiting altogether.
__device__ inline bool tree_exchange(TreePartView& v, const TreePart mine, TreeShared& sh) {
    constexpr int kPieces = kTreeParts * kShareHalves;
    constexpr int kPerLane = (kPieces + 63) / 64;  // pieces each lane of wavefront 0 collects
    v.tag += 1;
    const uint64_t tag48 = v.tag & ((1ULL << 48) - 1);
    __syncthreads();  // sh.xp of the previous exchange is no longer read
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        uint64_t* slot = v.shares + (v.tag & 1) * kPieces;
        if (lane < kShareHalves) {
            uint32_t w = mine.w[0];
#pragma unroll
            for (int i = 1; i < 6; ++i)
                w = (lane >> 1) == i ? mine.w[i] : w;
            const uint64_t piece = (w >> ((lane & 1) * 16)) & 0xFFFFu;
            __hip_atomic_store(slot + v.part * kShareHalves + lane, (tag48 << 16) | piece,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        bool ok = v.live;
        bool have[kPerLane];
        uint32_t got[kPerLane];
#pragma unroll
        for (int r = 0; r < kPerLane; ++r) {
            have[r] = lane + 64 * r >= kPieces;
            got[r] = 0;
        }
        int polls = 0;
        while (ok) {
            bool all = true;
#pragma unroll
            for (int r = 0; r < kPerLane; ++r) {
                if (!have[r]) {
                    const uint64_t x = __hip_atomic_load(slot + lane + 64 * r, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
                    if ((x >> 16) == tag48) {
                        got[r] = static_cast<uint32_t>(x & 0xFFFFu);
                        have[r] = true;
                    }
                }
                all = all && have[r];
            }
            if (__ballot(!all) == 0)
                break;
            if (++polls > v.spin_limit)
                ok = false;
            else
                __builtin_amdgcn_s_sleep(1);
        }
#pragma unroll
        for (int r = 0; r < kPerLane; ++r)
            if (ok && lane + 64 * r < kPieces)
                reinterpret_cast<uint16_t*>(sh.xp)[lane + 64 * r] = static_cast<uint16_t>(got[r]);
        if (lane == 0)
            sh.ok = ok ? 1 : 0;
    }
    __syncthreads();
    const bool ok = sh.ok != 0;
    v.live = v.live && ok;
    return ok;
}

// Row normaliser(s) of one node over the whole vocabulary: target row, and
// the draft row too when two_rows (one pass over both).
template <int DT, bool VEC, bool NT>
__device__ inline bool tree_norms(TreePartView& v, const void* prow, const void* qrow,
                                  bool two_rows, float inv_t, TreeShared& sh, float* mp,
                                  double* sp, float* mq, double* sq) {
    constexpr int W = Group<DT, VEC>::W;
    TreePart mine = part_zero();
    part_set_f(mine, 0, kNegMax);
    part_set_f(mine, 1, kNegMax);
    if (v.ng > 0) {
        OnlineNorm<W> np, nq;
        if (two_rows) {
            const void* const rows[2] = {v.sub(prow), v.sub(qrow)};
            tree_stream<DT, VEC, NT, 2, kTreeDepth2>(rows, v.ng, [&](int, bool in, const float (&z)[2][W]) {
                if (in) {
                    np.add(z[0], inv_t);
                    nq.add(z[1], inv_t);
                }
            });
            float m;
            double sum;
            nq.finish(sh, &m, &sum);
            part_set_f(mine, 1, m);
            part_set_d(mine, 4, sum);
        } else {
            const void* const rows[1] = {v.sub(prow)};
            tree_stream<DT, VEC, NT, 1, kTreeDepth1>(rows, v.ng, [&](int, bool in, const float (&z)[1][W]) {
                if (in)
                    np.add(z[0], inv_t);
            });
        }
        float m;
        double sum;
        np.finish(sh, &m, &sum);
        part_set_f(mine, 0, m);
        part_set_d(mine, 2, sum);
    }
    if (!tree_exchange(v, mine, sh))
        return false;
    merge_norm(sh, false, mp, sp);
    if (two_rows)
        merge_norm(sh, true, mq, sq);
    return true;
}

// Target argmax over the whole vocabulary (lowest index on ties); -1 when the
// row has no finite maximum, -2 when a partner went missing.
template <int DT, bool VEC, bool NT>
__device__ inline int tree_argmax(TreePartView& v, const void* row, TreeShared& sh) {
    constexpr int W = Group<DT, VEC>::W;
    TreePart mine = part_zero();
    part_set_f(mine, 0, -__builtin_huge_valf());
    mine.w[1] = 0x7fffffffu;
    if (v.ng > 0) {
        float bv = -__builtin_huge_valf();
        int bi = 0x7fffffff;
        const void* const rows[1] = {v.sub(row)};
        const int base = v.g0 * W;
        tree_stream<DT, VEC, NT, 1, kTreeDepth1>(rows, v.ng, [&](int g, bool in, const float (&z)[1][W]) {
#pragma unroll
            for (int e = 0; e < W; ++e)
                if (in && z[0][e] > bv) {
                    bv = z[0][e];
                    bi = base + g * W + e;
                }
        });
        float av;
        int ai;
        tree_block_argmax(bv, bi, sh, &av, &ai);
        part_set_f(mine, 0, av);
        mine.w[1] = static_cast<uint32_t>(ai);
    }
    if (!tree_exchange(v, mine, sh))
        return -2;
    float bv = part_f(sh.xp[0], 0);
    int bi = static_cast<int>(sh.xp[0].w[1]);
    for (int j = 1; j < kTreeParts; ++j) {
        const float av = part_f(sh.xp[j], 0);
        const int ai = static_cast<int>(sh.xp[j].w[1]);
        if (av > bv || (av == bv && ai < bi)) {
            bv = av;
            bi = ai;
        }
    }
    return bv > -__builtin_huge_valf() ? bi : -1;
}

// Tile sums of the row pair's weights over this part's run into ts (LDS), as
// the residual kernels form them, and the shares' totals in sh.xp (words 2-3).
// Returns false when a partner went missing.
template <int DT, bool VEC, bool NT>
__device__ inline bool tree_tile_pass(TreePartView& v, const SeqRows& s, float* ts, TreeShared& sh) {
    constexpr int W = Group<DT, VEC>::W;
    const int lane = threadIdx.x & 63;
    TreePart mine = part_zero();
    if (v.ng > 0) {
        const void* const rows[2] = {v.sub(s.prow), v.sub(s.qrow)};
        tree_stream<DT, VEC, NT, 2, kTreeDepth2>(rows, v.ng, [&](int g, bool in, const float (&z)[2][W]) {
            float r[W];
            if (!in) {
#pragma unroll
                for (int e = 0; e < W; ++e)
                    r[e] = 0.0f;
            } else if (s.p_only) {
#pragma unroll
                for (int e = 0; e < W; ++e)
                    r[e] = fast_exp2(__builtin_fmaf(scale_logit(z[0][e], s.inv_t), kLog2e, -s.mp));
            } else {
#pragma unroll
                for (int e = 0; e < W; ++e) {
                    const float pv = fast_exp2(__builtin_fmaf(scale_logit(z[0][e], s.inv_t), kLog2e, -s.mp));
                    const float qv = fast_exp2(__builtin_fmaf(scale_logit(z[1][e], s.inv_t), kLog2e, -s.mq));
                    r[e] = fmaxf(__builtin_fmaf(pv, s.ratio, -qv), 0.0f);
                }
            }
            const float tsum = tile_reduce(pairwise(r));
            if (lane == 0)
                ts[g / kTile] = tsum;
        });
        __syncthreads();
        double part = 0.0;
        for (int i = threadIdx.x; i < v.nt; i += kTreeBlock)
            part += static_cast<double>(ts[i]);
        part_set_d(mine, 2, tree_block_sum(part, sh));
    }
    return tree_exchange(v, mine, sh);
}

template <int DT, bool VEC, bool NT>
__global__ __launch_bounds__(kTreeBlock, 4) void tree_sample_kernel(TreeSampleArgs a) {
    constexpr int W = Group<DT, VEC>::W;
    extern __shared__ float lds_ts[];
    __shared__ TreeShared sh;
    const int tid = threadIdx.x;
    const int M = a.M, V = a.V;
    const int groups = V / W;
    const int ntiles = (groups + kTile - 1) / kTile;
    const int n_grp = gridDim.x / kTreeParts;
    const int grp = blockIdx.x / kTreeParts;

    TreePartView v;
    v.part = blockIdx.x % kTreeParts;
    {
        const int t0 = static_cast<int>(static_cast<long>(ntiles) * v.part / kTreeParts);
        const int t1 = static_cast<int>(static_cast<long>(ntiles) * (v.part + 1) / kTreeParts);
        v.g0 = t0 * kTile;
        v.ng = t1 > t0 ? min(t1 * kTile, groups) - v.g0 : 0;
        v.nt = t1 - t0;
    }
    v.W = W;
    v.dt = DT;
    v.shares = a.shares + static_cast<size_t>(grp) * 2 * kTreeParts * kShareHalves;
    // This launch's number: one more than the launches finished before it.
    const uint64_t call = __hip_atomic_load(a.ctl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
    v.tag = call << 20;
    v.spin_limit = a.spin_limit;
    v.live = true;

    for (int b = grp; b < a.B; b += n_grp) {
        const int n = a.n_nodes[b];
        // Structure, tokens and temperature (every part reads them).
        if (tid == 0)
            sh.flag = 0;
        __syncthreads();
        const bool n_ok = n >= 1 && n <= M;
        for (int i = tid; n_ok && i < n; i += kTreeBlock) {
            const int pr = a.parent[static_cast<size_t>(b) * M + i];
            const int tk = a.token[static_cast<size_t>(b) * M + i];
            sh.parent[i] = pr;
            sh.token[i] = tk;
            const bool ok = i == 0 ? pr == -1 : (pr >= 0 && pr < i && tk >= 0 && tk < V);
            if (!ok)
                atomicOr(&sh.flag, 1);
        }
        float inv_t = 0.0f;
        const int mode = temperature_mode(a.temperature[b], &inv_t);
        __syncthreads();
        bool bad = !n_ok || sh.flag != 0 || mode < 0 || !v.live;

        const size_t row_base = static_cast<size_t>(b) * M;
        auto prow = [&](int u) { return row_ptr(a.target, DT, row_base + u, V); };
        auto qrow = [&](int u) { return row_ptr(a.draft, DT, row_base + u, V); };
        int u = 0, L = 0, extra = -1;
        bool draw_here = false;  // this part draws the extra token
        int owner = 0;           // the part that draws it
        if (!bad && mode == 0) {
            // T = 0: step to the lowest-index child holding the target argmax.
            for (;;) {
                const int am = tree_argmax<DT, VEC, NT>(v, prow(u), sh);
                if (am < 0) {
                    bad = true;
                    break;
                }
                node_set(sh, n, [&](int i) { return i > u && sh.parent[i] == u && sh.token[i] == am; });
                const int next = node_set_next(sh, u + 1, -1);
                if (next < 0) {
                    extra = am;
                    break;
                }
                if (tid == 0)
                    sh.path[L] = next;
                ++L;
                u = next;
            }
        } else if (!bad) {
            float mp = 0.0f, mq = 0.0f;
            double sp = 0.0, sq = 0.0;
            int s = n;  // the child of u to test next (n: none left)
            // Child c's token logits in x's rows, loaded a pass ahead of its
            // test as raw bits and converted only at the test: a conversion
            // here would wait for the loads before the pass's own loads leave.
            uint32_t zs_p_bits = 0, zs_q_bits = 0;
            auto fetch = [&](int x, int c) {
                if (c < n) {
                    const int t = sh.token[c];
                    zs_p_bits = load_logit_bits(prow(x), DT, t);
                    zs_q_bits = load_logit_bits(qrow(x), DT, t);
                }
            };
            // Arrival at x: its children (sh.nodes), the first one's logits,
            // and the normalisers of x's rows: the draft row's only when x has
            // children to test, then in the same pass.
            auto arrive = [&](int x) {
                node_set(sh, n, [&](int i) { return i > x && sh.parent[i] == x; });
                s = node_set_next(sh, x + 1, n);
                const bool kids = s < n;
                fetch(x, s);
                if (!tree_norms<DT, VEC, NT>(v, prow(x), qrow(x), kids, inv_t, sh, &mp, &sp, &mq, &sq))
                    return false;
                return sp > 0.0 && (!kids || sq > 0.0);
            };
            bad = !arrive(u);
            double c = 0.0, Z = 1.0;
            bool ts_current = false;  // lds_ts holds the tile sums of the current (c, Z)
            while (!bad && s < n) {
                // The accept test of child s, in fp64 (every thread computes it).
                const double lse_p = (static_cast<double>(mp) + log2(sp)) / static_cast<double>(kLog2e);
                const double lse_q = (static_cast<double>(mq) + log2(sq)) / static_cast<double>(kLog2e);
                const double lp = static_cast<double>(scale_logit(logit_of_bits(zs_p_bits, DT), inv_t)) - lse_p;
                const double lq = static_cast<double>(scale_logit(logit_of_bits(zs_q_bits, DT), inv_t)) - lse_q;
                double lpi = lp;
                if (c > 0.0) {
                    const double d = exp(lp) - c * exp(lq);
                    lpi = d > 0.0 ? log(d) - log(Z) : -__builtin_huge_val();
                }
                const Words4 w = verify_block(a.seed, a.offset, static_cast<uint32_t>(b),
                                              static_cast<uint32_t>(s - 1));
                const double log_u = log(static_cast<double>(uniform24(w.w0)));
                if (log_u < lpi - lq) {
                    if (tid == 0)
                        sh.path[L] = s;
                    ++L;
                    u = s;
                    c = 0.0;
                    Z = 1.0;
                    ts_current = false;
                    bad = !arrive(u);
                    continue;
                }
                // Rejected: the residual against q_u, in closed form; the next
                // child's logits load behind its pass.
                const int s_next = node_set_next(sh, s + 1, n);
                fetch(u, s_next);
                const double c2 = c + Z;
                SeqRows rows;
                rows.prow = prow(u);
                rows.qrow = qrow(u);
                rows.p_only = false;
                rows.inv_t = inv_t;
                rows.mp = mp;
                rows.mq = mq;
                rows.ratio = static_cast<float>(sq / (c2 * sp));
                if (!tree_tile_pass<DT, VEC, NT>(v, rows, lds_ts, sh)) {
                    bad = true;
                    break;
                }
                double tot = 0.0;
                for (int j = 0; j < kTreeParts; ++j)
                    tot += part_d(sh.xp[j], 2);
                const double Z2 = c2 / sq * tot;
                if (Z2 > 0.0) {
                    c = c2;
                    Z = Z2;
                    ts_current = true;
                    if (tid < kTreeParts)
                        sh.tot_keep[tid] = part_d(sh.xp[tid], 2);
                } else {
                    ts_current = false;  // an empty residual (rounding): pi stays
                }
                s = s_next;
            }
            if (!bad) {
                SeqRows rows;
                rows.prow = prow(u);
                rows.qrow = c > 0.0 ? qrow(u) : prow(u);
                rows.p_only = !(c > 0.0);
                rows.inv_t = inv_t;
                rows.mp = mp;
                rows.mq = mq;
                rows.ratio = c > 0.0 ? static_cast<float>(sq / (c * sp)) : 1.0f;
                if (!ts_current) {
                    if (!tree_tile_pass<DT, VEC, NT>(v, rows, lds_ts, sh))
                        bad = true;
                    else if (tid < kTreeParts)
                        sh.tot_keep[tid] = part_d(sh.xp[tid], 2);
                }
                __syncthreads();  // sh.tot_keep
                if (!bad) {
                    // The draw position over the parts' totals in part order;
                    // past the total (rounding only) it falls to the last part
                    // with mass, which then takes its last positive element.
                    double S = 0.0;
                    for (int j = 0; j < kTreeParts; ++j)
                        S += sh.tot_keep[j];
                    const Words4 w = verify_block(a.seed, a.offset, static_cast<uint32_t>(b),
                                                  static_cast<uint32_t>(L));
                    const float uu = uniform24(w.w1);
                    if (S > 0.0) {
                        const double tau = static_cast<double>(uu) * S;
                        int last = -1;
                        double P = 0.0, P_owner = 0.0, P_last = 0.0;
                        owner = -1;
                        for (int j = 0; j < kTreeParts; ++j) {
                            const double tj = sh.tot_keep[j];
                            if (tj > 0.0) {
                                if (owner < 0 && P + tj > tau) {
                                    owner = j;
                                    P_owner = P;
                                }
                                last = j;
                                P_last = P;
                            }
                            P += tj;
                        }
                        if (owner < 0) {
                            owner = last;
                            P_owner = P_last;
                        }
                        draw_here = owner == v.part;
                        if (draw_here && tid < 64) {
                            SeqRows local = rows;
                            local.prow = v.sub(rows.prow);
                            local.qrow = v.sub(rows.qrow);
                            const int tok = draw_at<DT, VEC, NT>(local, tau - P_owner, lds_ts, v.nt, v.ng);
                            if (tid == 0)
                                sh.decision = tok + v.g0 * W;
                        }
                    } else {
                        // Empty residual (rounding only): part 0 draws from p.
                        draw_here = v.part == 0;
                        if (draw_here && tid < 64) {
                            const int tok = draw_p_fallback<DT, VEC, NT>(rows, uu, ntiles, groups);
                            if (tid == 0)
                                sh.decision = tok;
                        }
                    }
                    __syncthreads();
                    extra = sh.decision;
                }
            }
        }
        // The drawing part hands its token to part 0 (every part knows the
        // owner: it follows from the merged totals).
        if (!bad && mode != 0 && owner > 0) {
            TreePart mine = part_zero();
            mine.w[0] = static_cast<uint32_t>(draw_here ? extra : 0);
            if (!tree_exchange(v, mine, sh))
                bad = true;
            else
                extra = static_cast<int>(sh.xp[owner].w[0]);
        }
        // Part 0 writes the outcome: -2 once it or a partner gave up waiting,
        // -1 for invalid input.
        const bool gave_up = !v.live;
        const bool fail = bad || gave_up;
        __syncthreads();
        if (v.part == 0) {
            int32_t* path_out = a.out_path + static_cast<size_t>(b) * M;
            for (int i = tid; i < M; i += kTreeBlock)
                path_out[i] = !fail && i < L ? sh.path[i] : -1;
            if (tid == 0) {
                a.out_length[b] = gave_up ? -2 : (bad ? -1 : L);
                a.out_extra[b] = fail ? -1 : extra;
                if (gave_up)
                    __hip_atomic_fetch_add(a.ctl + 2, 1ULL, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __syncthreads();
    }
    // The last workgroup to finish advances the launch counter. Every
    // workgroup read it at its start, so no part of this launch can see the
    // new value; the next launch on the stream starts after this one ends.
    if (tid == 0) {
        const uint64_t done = __hip_atomic_fetch_add(a.ctl + 1, 1ULL, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (done + 1 == gridDim.x) {
            __hip_atomic_store(a.ctl + 1, 0ULL, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.ctl, call, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int DT, bool VEC>
hipError_t tree_sample_capacity_typed(int* blocks) {
    constexpr bool NT = VEC;
    constexpr int W = Group<DT, VEC>::W;
    (void)W;
    int per_cu = 0;
    // The dynamic LDS of the largest run is at most 16 KiB for any vocabulary
    // up to 2^22 groups; capacity is taken at that size.
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, reinterpret_cast<const void*>(tree_sample_kernel<DT, VEC, NT>), kTreeBlock,
        kTreeLdsBytes);
    if (e != hipSuccess)
        return e;
    int dev = 0, cus = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess)
        return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
        return e;
    *blocks = per_cu * cus;
    return hipSuccess;
}

template <int DT, bool VEC>
hipError_t launch_tree_sample_typed(int n_groups, const TreeSampleArgs& args, hipStream_t stream) {
    constexpr bool NT = VEC;
    constexpr int W = Group<DT, VEC>::W;
    const int ntiles = (args.V / W + kTile - 1) / kTile;
    const int run_tiles = (ntiles + kTreeParts - 1) / kTreeParts;
    const size_t lds = static_cast<size_t>(run_tiles) * sizeof(float);
    if (lds > kTreeLdsBytes)
        return hipErrorInvalidValue;
    tree_sample_kernel<DT, VEC, NT><<<dim3(static_cast<unsigned>(n_groups * kTreeParts)),
                                       dim3(kTreeBlock), lds, stream>>>(args);
    return hipGetLastError();
}

// Largest LDS request of the fused draw with its group sums (the CU has
// 160 KiB; a workgroup of it is alone on its CU either way).
constexpr size_t kFusedGsMaxBytes = 144 * 1024;

// The kernel with group sums may ask for up to kFusedGsMaxBytes of dynamic
// LDS: raised once per instantiation; without it the draw recomputes them.
template <int DT, bool VEC, bool NT>
bool fused_gs_allowed() {
    static const bool ok =
        hipFuncSetAttribute(reinterpret_cast<const void*>(
                                residual_fused_kernel<DT, VEC, NT, kFusedBlock, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(kFusedGsMaxBytes)) == hipSuccess;
    return ok;
}

template <int DT, bool VEC, int U>
hipError_t launch_typed(const Shape& sh, int nsplit, int tiles_per_row, const void* draft,
                        const void* target, const SeqState* seq, float* tile_sums,
                        int32_t* out_tok, const AcceptArgs* acc, hipStream_t stream,
                        const LaunchEvents& ev) {
    constexpr bool NT = VEC;
    constexpr int W = Group<DT, VEC>::W;
    if (sh.batch == 0)
        return hipSuccess;
    const int groups = sh.vocab / W;
    const int ntiles = (groups + kTile - 1) / kTile;
    if (nsplit == 0) {
        // Two tiles in flight per wavefront: 12 wavefronts keep 48 KiB in
        // flight per workgroup. The group sums join the tile sums in LDS when
        // they fit.
        const size_t ts_bytes = static_cast<size_t>(ntiles) * sizeof(float);
        const size_t gs_bytes = ts_bytes * (1 + kTile);
        if (gs_bytes <= kFusedGsMaxBytes && fused_gs_allowed<DT, VEC, NT>())
            return launch(residual_fused_kernel<DT, VEC, NT, kFusedBlock, true>,
                          dim3(static_cast<unsigned>(sh.batch)), dim3(kFusedBlock), gs_bytes,
                          stream, ev, draft, target, sh.gamma, sh.vocab, ntiles, seq, out_tok);
        return launch(residual_fused_kernel<DT, VEC, NT, kFusedBlock, false>,
                      dim3(static_cast<unsigned>(sh.batch)), dim3(kFusedBlock), ts_bytes, stream,
                      ev, draft, target, sh.gamma, sh.vocab, ntiles, seq, out_tok);
    }
    // Timing the split pair: the tile kernel's start to the locate kernel's stop.
    const int per = (ntiles + nsplit - 1) / nsplit;
    const dim3 tgrid(static_cast<unsigned>(sh.batch), static_cast<unsigned>(nsplit));
    const LaunchEvents tev{ev.start, nullptr};
    const hipError_t e =
        acc ? launch(residual_tiles_kernel<DT, VEC, U, NT, true>, tgrid, dim3(kBlock), 0, stream,
                     tev, draft, target, sh.gamma, sh.vocab, ntiles, per, tiles_per_row, seq,
                     tile_sums, *acc)
            : launch(residual_tiles_kernel<DT, VEC, U, NT, false>, tgrid, dim3(kBlock), 0, stream,
                     tev, draft, target, sh.gamma, sh.vocab, ntiles, per, tiles_per_row, seq,
                     tile_sums, AcceptArgs{});
    if (e != hipSuccess)
        return e;
    return launch(residual_locate_kernel<DT, VEC, NT>, dim3(static_cast<unsigned>(sh.batch)),
                  dim3(64), 0, stream, LaunchEvents{nullptr, ev.stop}, draft, target, sh.gamma,
                  sh.vocab, ntiles, tiles_per_row, seq, tile_sums, out_tok);
}

template <int DT, bool VEC>
hipError_t launch_unroll(const Shape& sh, int nsplit, int unroll, int tiles_per_row,
                         const void* draft, const void* target, const SeqState* seq,
                         float* tile_sums, int32_t* out_tok, const AcceptArgs* acc,
                         hipStream_t stream, const LaunchEvents& ev) {
    if (unroll == 2)
        return launch_typed<DT, VEC, 2>(sh, nsplit, tiles_per_row, draft, target, seq, tile_sums,
                                        out_tok, acc, stream, ev);
    return launch_typed<DT, VEC, 4>(sh, nsplit, tiles_per_row, draft, target, seq, tile_sums,
                                    out_tok, acc, stream, ev);
}

}  // namespace

int residual_tiles_per_row(int vocab) { return (vocab + kTile - 1) / kTile; }

int tree_sample_parts() { return kTreeParts; }

int tree_sample_default_spin_limit() { return kTreeSpinLimit; }

bool tree_sample_fits(int vocab, int dtype) {
    // The element path (W = 1) has the most tiles.
    (void)dtype;
    const long run_tiles = ((static_cast<long>(vocab) + kTile - 1) / kTile + kTreeParts - 1) / kTreeParts;
    return run_tiles * static_cast<long>(sizeof(float)) <= static_cast<long>(kTreeLdsBytes);
}

size_t tree_sample_group_bytes() { return 2 * kTreeParts * kShareHalves * sizeof(uint64_t); }

hipError_t tree_sample_max_groups(int dtype, int* out_groups) {
    int a = 0, b = 0;
    hipError_t e = dtype == kBF16 ? tree_sample_capacity_typed<kBF16, true>(&a)
                                  : tree_sample_capacity_typed<kF32, true>(&a);
    if (e != hipSuccess)
        return e;
    e = dtype == kBF16 ? tree_sample_capacity_typed<kBF16, false>(&b)
                       : tree_sample_capacity_typed<kF32, false>(&b);
    if (e != hipSuccess)
        return e;
    *out_groups = std::min(a, b) / kTreeParts;
    return hipSuccess;
}

hipError_t launch_tree_sample(int batch, int max_nodes, int vocab, int dtype, bool vec,
                              const int32_t* parent, const int32_t* token, const int32_t* n_nodes,
                              const void* draft, const void* target, const float* temperature,
                              uint64_t seed, uint64_t offset, int32_t* out_length,
                              int32_t* out_path, int32_t* out_extra, uint64_t* shares,
                              uint64_t* ctl, int spin_limit, int n_groups, hipStream_t stream) {
    if (batch == 0)
        return hipSuccess;
    if (n_groups < 1 || spin_limit < 0 || !ctl)
        return hipErrorInvalidValue;
    const TreeSampleArgs args{parent, token, n_nodes, draft, target, temperature, batch,
                              max_nodes, vocab, seed, offset, out_length, out_path, out_extra,
                              shares, ctl, spin_limit};
    const int g = std::min(n_groups, batch);
    if (dtype == kBF16)
        return vec ? launch_tree_sample_typed<kBF16, true>(g, args, stream)
                   : launch_tree_sample_typed<kBF16, false>(g, args, stream);
    return vec ? launch_tree_sample_typed<kF32, true>(g, args, stream)
               : launch_tree_sample_typed<kF32, false>(g, args, stream);
}

int residual_fused_max_tiles() { return kResidualFusedMaxTiles; }

hipError_t launch_residual(const Shape& s, bool vec, int nsplit, int unroll, const void* draft,
                           const void* target, const SeqState* seq, float* tile_sums,
                           int32_t* out_tok, const AcceptArgs* acc, hipStream_t stream,
                           const LaunchEvents& ev) {
    if (nsplit < 0 || nsplit > kMaxSplit || (acc && nsplit == 0))
        return hipErrorInvalidValue;
    if (nsplit == 0 && residual_tiles_per_row(s.vocab) > kResidualFusedMaxTiles)
        return hipErrorInvalidValue;
    // Tile sums are laid out with the element-path tile count, which bounds the
    // 16-byte-group tile count.
    const int tiles = residual_tiles_per_row(s.vocab);
    if (s.dtype == kBF16)
        return vec ? launch_unroll<kBF16, true>(s, nsplit, unroll, tiles, draft, target, seq,
                                                tile_sums, out_tok, acc, stream, ev)
                   : launch_unroll<kBF16, false>(s, nsplit, unroll, tiles, draft, target, seq,
                                                 tile_sums, out_tok, acc, stream, ev);
    return vec ? launch_unroll<kF32, true>(s, nsplit, unroll, tiles, draft, target, seq, tile_sums,
                                           out_tok, acc, stream, ev)
               : launch_unroll<kF32, false>(s, nsplit, unroll, tiles, draft, target, seq,
                                            tile_sums, out_tok, acc, stream, ev);
}

}  // namespace specv
