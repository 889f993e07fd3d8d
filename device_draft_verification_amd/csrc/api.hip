// The C ABI (include/spec_verify.h): context, workspace, argument checks and
// the launch sequence row-normaliser -> accept -> residual on one stream.
// Nothing here synchronises the host except spec_verify_read_timing and
// spec_verify_destroy.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <new>
#include <vector>

#include "launch.hpp"
#include "outcome.hpp"
#include "spec_verify.h"

using namespace specv;

namespace {

// Launch geometry, a function of the shape (and the tuning variables).
struct Geometry {
    int nsplit_rows = 1;      // vocabulary splits of the row-normaliser kernel
    int row_unroll = 8;       // 16-byte groups in flight per thread in that kernel
    bool row_nontemporal = true;
    int nsplit_residual = 1;  // vocabulary splits of the residual kernel (0: fused)
    int residual_unroll = 4;  // tiles per batch per wavefront in that kernel
    int nsplit_outcome = 1;   // vocabulary splits of the outcome kernel
};

// The arrays one verification call works in (all inside one buffer).
struct Workspace {
    Partial* part = nullptr;
    float* gathered = nullptr;
    RowNorm* rn = nullptr;
    double* lse = nullptr;
    SeqState* seq = nullptr;
    float* tile_sums = nullptr;
    OutcomeWork outcome{};
};

}  // namespace

struct spec_verify_ctx {
    Shape shape{};
    hipStream_t stream = nullptr;
    int device = 0;
    Geometry geo{};

    void* ws_base = nullptr;
    Workspace ws{};
    bool have_verified = false;

    int timing_slots = 0;
    int timing_count = 0;
    std::vector<hipEvent_t> events;  // per slot: start and stop of each of the three steps
};

namespace {

// Workgroup counts per launch: the row kernel wants several waves of
// workgroups over the 256 CUs so the last wave is short; the residual kernel's
// workgroups are short-lived, so fewer, longer ones.
constexpr long kRowTargetBlocks = 12288;
constexpr long kRowFillBlocks = 1024;  // four row workgroups per CU
constexpr long kResidualTargetBlocks = 4096;
// Outcome splits: as many as keep the whole grid within about one wave of
// resident workgroups (rounded down); larger batches keep one split. At
// B = 64, V = 128 256 (384 pairs), 2 splits took 54 us per call, 3, 4 and 6
// splits 62, 58 and 65 us: a partly filled second wave costs more than
// longer splits.
constexpr long kOutcomeWaveBlocks = 1024;
constexpr int kResidualFusedMinBatch = 128;

int env_int(const char* name, int fallback) {
    const char* v = std::getenv(name);
    if (!v || !*v)
        return fallback;
    return std::atoi(v);
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int group_width(int dtype) { return dtype == SPEC_BF16 ? 8 : 4; }

// Splits per row: about target_blocks workgroups in total, at least
// min_groups 16-byte groups per split, at most kMaxSplit.
int choose_split(long rows, long vocab, int dtype, long target_blocks, long min_groups) {
    if (rows <= 0)
        return 1;
    const long groups = vocab / group_width(dtype);
    long n = (target_blocks + rows - 1) / rows;
    const long by_size = std::max(1L, groups / min_groups);
    n = std::min(n, by_size);
    n = std::max(1L, std::min(n, static_cast<long>(kMaxSplit)));
    return static_cast<int>(n);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool shape_valid(const Shape& s) {
    if (s.batch < 0 || s.gamma < 0 || s.vocab < 1 || (s.dtype != SPEC_F32 && s.dtype != SPEC_BF16))
        return false;
    const long rows = static_cast<long>(s.batch) * (2L * s.gamma + 1);
    return rows < (1L << 31) && static_cast<long>(s.batch) * (s.gamma + 1) < (1L << 31);
}

// The launch geometry of a shape (host arithmetic and the tuning variables
// only). False when a dispatch would hold 2^32 work-items or more.
bool compute_geometry(const Shape& s, Geometry* out) {
    Geometry g;
    const int batch = s.batch, gamma = s.gamma, vocab = s.vocab, dtype = s.dtype;
    const long rows = static_cast<long>(batch) * (2L * gamma + 1);
    g.nsplit_rows = choose_split(rows, vocab, dtype, kRowTargetBlocks, 4L * kBlock);
    g.nsplit_residual = choose_split(batch, vocab, dtype, kResidualTargetBlocks, 16L * 64);
    const long pairs = static_cast<long>(batch) * (gamma + 1);
    {
        const long by_size = std::max(1L, vocab / group_width(dtype) / (16L * 64));
        long n = pairs > 0 ? kOutcomeWaveBlocks / pairs : 1;
        n = std::max(1L, std::min({n, by_size, static_cast<long>(kOutcomeMaxSplit)}));
        g.nsplit_outcome = static_cast<int>(n);
    }
    const int oo = env_int("SPEC_VERIFY_OUTCOME_SPLIT", 0);
    if (oo > 0)
        g.nsplit_outcome = std::min(oo, kOutcomeMaxSplit);
    const int o1 = env_int("SPEC_VERIFY_ROW_SPLIT", 0), o3 = env_int("SPEC_VERIFY_RESIDUAL_SPLIT", 0);
    if (o1 > 0)
        g.nsplit_rows = std::min(o1, kMaxSplit);
    if (o3 > 0)
        g.nsplit_residual = std::min(o3, kMaxSplit);
    const int ou = env_int("SPEC_VERIFY_ROW_UNROLL", 0);
    if (ou == 2 || ou == 4 || ou == 8)
        g.row_unroll = ou;
    // Row splits are whole batch strides (unroll x kBlock groups): more splits
    // than strides would only add empty splits for the accept kernel to merge.
    // Unless the rows alone are too few to give every CU a few workgroups, a
    // split also keeps about three batches per thread, so that a thread's
    // loads overlap each other and the block's closing reduction is paid for
    // by more than one batch (at B = 64, V = 128256: 2 splits instead of 8,
    // 57.1 -> 51.6 us per call).
    {
        const long stride = static_cast<long>(g.row_unroll) * kBlock;
        const long strides = std::max(1L, (vocab / group_width(dtype) + stride - 1) / stride);
        long n = std::min<long>(g.nsplit_rows, strides);
        if (o1 <= 0) {
            const long fill = rows > 0 ? (kRowFillBlocks + rows - 1) / rows : 1;
            n = std::min(n, std::max(fill, std::max(1L, strides / 3)));
        }
        g.nsplit_rows = static_cast<int>(n);
    }
    g.row_nontemporal = env_int("SPEC_VERIFY_ROW_NT", g.row_nontemporal ? 1 : 0) != 0;
    const int ru = env_int("SPEC_VERIFY_RESIDUAL_UNROLL", 0);
    if (ru == 2 || ru == 4)
        g.residual_unroll = ru;
    // With at least half as many sequences as CUs, one workgroup per sequence
    // (the fused residual kernel) fills the GPU by itself.
    const bool fused_fits = residual_tiles_per_row(vocab) <= residual_fused_max_tiles();
    int fused = batch >= kResidualFusedMinBatch && fused_fits ? 1 : 0;
    fused = env_int("SPEC_VERIFY_RESIDUAL_FUSED", fused);
    if (fused && fused_fits && o3 <= 0)
        g.nsplit_residual = 0;
    // A dispatch holds fewer than 2^32 work-items.
    const long long limit = 1LL << 32;
    if (static_cast<long long>(rows) * g.nsplit_rows * kBlock >= limit ||
        static_cast<long long>(batch) * std::max(g.nsplit_residual, 1) * kBlock >= limit ||
        static_cast<long long>(pairs) * g.nsplit_outcome * kBlock >= limit)
        return false;
    *out = g;
    return true;
}

// Bytes of the workspace of a shape and geometry (256-byte aligned
// sub-arrays; the outcome arrays only when asked for). With base non-null,
// also fills *ws with the sub-arrays' addresses in that buffer.
size_t layout_workspace(const Shape& s, const Geometry& g, bool with_outcome, char* base,
                        Workspace* ws) {
    const size_t rows = static_cast<size_t>(s.batch) * (2 * static_cast<size_t>(s.gamma) + 1);
    const size_t n_part = rows * static_cast<size_t>(g.nsplit_rows);
    size_t off = 0;
    const size_t o_part = off; off = align_up(off + n_part * sizeof(Partial), 256);
    const size_t o_rn = off;   off = align_up(off + rows * sizeof(RowNorm), 256);
    const size_t o_ga = off;   off = align_up(off + rows * sizeof(float), 256);
    const size_t o_lse = off;  off = align_up(off + rows * sizeof(double), 256);
    const size_t o_seq = off;  off = align_up(off + static_cast<size_t>(s.batch) * sizeof(SeqState), 256);
    const size_t o_ts = off;
    if (g.nsplit_residual > 0)  // the fused draw keeps its tile sums in LDS
        off = align_up(off + static_cast<size_t>(s.batch) * residual_tiles_per_row(s.vocab) * sizeof(float), 256);
    size_t o_oc = off, o_os = off;
    if (with_outcome) {
        const size_t n_oc = static_cast<size_t>(s.batch) * (s.gamma + 1) * g.nsplit_outcome;
        o_oc = off; off = align_up(off + n_oc * kOutcomeMaxF * sizeof(Cand), 256);
        o_os = off; off = align_up(off + n_oc * sizeof(double), 256);
    }
    if (base) {
        ws->part = reinterpret_cast<Partial*>(base + o_part);
        ws->rn = reinterpret_cast<RowNorm*>(base + o_rn);
        ws->gathered = reinterpret_cast<float*>(base + o_ga);
        ws->lse = reinterpret_cast<double*>(base + o_lse);
        ws->seq = reinterpret_cast<SeqState*>(base + o_seq);
        ws->tile_sums = reinterpret_cast<float*>(base + o_ts);
        ws->outcome.cand = with_outcome ? reinterpret_cast<Cand*>(base + o_oc) : nullptr;
        ws->outcome.sums = with_outcome ? reinterpret_cast<double*>(base + o_os) : nullptr;
    }
    return off;
}

}  // namespace

extern "C" {

const char* spec_verify_strerror(int code) {
    switch (code) {
    case SPEC_OK: return "ok";
    case SPEC_EINVAL: return "invalid argument";
    case SPEC_EHIP: return "HIP runtime error";
    case SPEC_ENOMEM: return "out of device memory";
    case SPEC_ESTATE: return "context in the wrong state for this call";
    case SPEC_ESCRATCH: return "the shape's workspace exceeds the fixed scratch array";
    default: return "unknown status";
    }
}

int spec_verify_init(int batch, int gamma, int vocab, int dtype, void* hip_stream,
                     spec_verify_ctx** out_ctx) {
    if (!out_ctx)
        return SPEC_EINVAL;
    *out_ctx = nullptr;
    const Shape shape{batch, gamma, vocab, dtype};
    Geometry geo;
    if (!shape_valid(shape) || !compute_geometry(shape, &geo))
        return SPEC_EINVAL;

    spec_verify_ctx* ctx = new (std::nothrow) spec_verify_ctx();
    if (!ctx)
        return SPEC_ENOMEM;
    ctx->shape = shape;
    ctx->geo = geo;
    ctx->stream = static_cast<hipStream_t>(hip_stream);
    if (hipGetDevice(&ctx->device) != hipSuccess) {
        delete ctx;
        return SPEC_EHIP;
    }
    // Workspace: one allocation, 256-byte aligned sub-arrays.
    const size_t total = std::max<size_t>(layout_workspace(shape, geo, true, nullptr, nullptr), 256);
    if (hipMalloc(&ctx->ws_base, total) != hipSuccess) {
        delete ctx;
        return SPEC_ENOMEM;
    }
    layout_workspace(shape, geo, true, static_cast<char*>(ctx->ws_base), &ctx->ws);
    // Defined contents before the first call (every entry is rewritten by it).
    if (hipMemset(ctx->ws_base, 0, total) != hipSuccess) {
        (void)hipFree(ctx->ws_base);
        delete ctx;
        return SPEC_EHIP;
    }
    *out_ctx = ctx;
    return SPEC_OK;
}

int spec_verify_set_stream(spec_verify_ctx* ctx, void* hip_stream) {
    if (!ctx)
        return SPEC_EINVAL;
    ctx->stream = static_cast<hipStream_t>(hip_stream);
    return SPEC_OK;
}

}  // extern "C"

namespace {

// Host-checkable arguments of a verification call (batch > 0).
bool verify_args_valid(const Shape& s, const void* logits_draft, const void* logits_target,
                       const int32_t* draft_tokens, const float* temperature,
                       const int32_t* out_accept_len, const int32_t* out_tokens) {
    const size_t esz = s.dtype == SPEC_BF16 ? 2 : 4;
    if (!logits_target || !temperature || !out_accept_len || !out_tokens)
        return false;
    if (s.gamma > 0 && (!logits_draft || !draft_tokens))
        return false;
    return aligned(logits_target, esz) && (!logits_draft || aligned(logits_draft, esz)) &&
           aligned(temperature, 4) && aligned(out_accept_len, 4) && aligned(out_tokens, 4) &&
           (!draft_tokens || aligned(draft_tokens, 4));
}

// The verification call on a shape, its geometry and a workspace; the
// Philox offset is `offset`, or the device word *offset_dev when that is
// non-null. Timing events may be null. Launches kernels only.
int verify_launch(const Shape& s, const Geometry& geo, const Workspace& ws, hipStream_t st,
                  const void* logits_draft, const void* logits_target,
                  const int32_t* draft_tokens, const float* temperature, uint64_t seed,
                  uint64_t offset, const uint64_t* offset_dev, int32_t* out_accept_len,
                  int32_t* out_tokens, const LaunchEvents& ev_row, const LaunchEvents& ev_acc,
                  const LaunchEvents& ev_res) {
    if (s.batch == 0)
        return SPEC_OK;
    if (!verify_args_valid(s, logits_draft, logits_target, draft_tokens, temperature,
                           out_accept_len, out_tokens))
        return SPEC_EINVAL;
    if (s.gamma == 0)
        logits_draft = logits_target;  // never read; keeps the kernels' pointers valid

    // 16-byte groups need every row start 16-byte aligned.
    const bool vec = (s.vocab % group_width(s.dtype)) == 0 && aligned(logits_target, 16) &&
                     aligned(logits_draft, 16);
    const RowTuning tu{geo.nsplit_rows, geo.row_unroll, geo.row_nontemporal};
    if (launch_row_norm(s, vec, tu, logits_draft, logits_target, temperature, draft_tokens,
                        ws.part, ws.gathered, st, ev_row) != hipSuccess)
        return SPEC_EHIP;
    const AcceptArgs acc{draft_tokens, temperature, s.gamma, s.vocab, geo.nsplit_rows, seed,
                         offset, offset_dev, ws.part, ws.gathered, ws.rn, ws.lse,
                         ws.seq, out_accept_len, out_tokens};
    // On the tile path (small batches) the tile kernel runs the accept step
    // itself, which saves a launch; the fused draw needs the accept kernel.
    const bool fold = geo.nsplit_residual > 0;
    if (!fold && launch_accept(s.batch, acc, st, ev_acc) != hipSuccess)
        return SPEC_EHIP;
    if (launch_residual(s, vec, geo.nsplit_residual, geo.residual_unroll, logits_draft,
                        logits_target, ws.seq, ws.tile_sums, out_tokens, fold ? &acc : nullptr,
                        st, ev_res) != hipSuccess)
        return SPEC_EHIP;
    return SPEC_OK;
}

// The workspace of spec_verify_noalloc: a fixed device array, zero at load,
// one copy per device. Host code never passes its name to a kernel (on the
// host the name is only a stand-in); it uses the device address that
// hipGetSymbolAddress returns, looked up once per device with that device
// current and kept here.
constexpr size_t kScratchBytes = SPEC_VERIFY_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return SPEC_EHIP;
    if (dev < 0 || dev >= kMaxDevices)
        return SPEC_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return SPEC_EHIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SPEC_OK;
}

// The verification call on a context.
int verify_impl(spec_verify_ctx* ctx, const void* logits_draft, const void* logits_target,
                const int32_t* draft_tokens, const float* temperature, uint64_t seed,
                uint64_t offset, const uint64_t* offset_dev, int32_t* out_accept_len,
                int32_t* out_tokens) {
    if (!ctx)
        return SPEC_EINVAL;
    // Timing mode: each step's start and stop events ride on its kernels'
    // own dispatches, so they time the kernels alone.
    if (ctx->shape.batch == 0)
        return SPEC_OK;
    if (!verify_args_valid(ctx->shape, logits_draft, logits_target, draft_tokens, temperature,
                           out_accept_len, out_tokens))
        return SPEC_EINVAL;
    LaunchEvents ev_row, ev_acc, ev_res;
    if (ctx->timing_slots > 0) {
        hipEvent_t* ev = &ctx->events[static_cast<size_t>(ctx->timing_count % ctx->timing_slots) * 6];
        ++ctx->timing_count;
        ev_row = LaunchEvents{ev[0], ev[1]};
        ev_acc = LaunchEvents{ev[2], ev[3]};
        ev_res = LaunchEvents{ev[4], ev[5]};
    }
    const int rc = verify_launch(ctx->shape, ctx->geo, ctx->ws, ctx->stream, logits_draft,
                                 logits_target, draft_tokens, temperature, seed, offset,
                                 offset_dev, out_accept_len, out_tokens, ev_row, ev_acc, ev_res);
    if (rc == SPEC_OK)
        ctx->have_verified = true;
    return rc;
}

}  // namespace

extern "C" {

int spec_verify(spec_verify_ctx* ctx, const void* logits_draft, const void* logits_target,
                const int32_t* draft_tokens, const float* temperature, uint64_t seed,
                uint64_t offset, int32_t* out_accept_len, int32_t* out_tokens) {
    return verify_impl(ctx, logits_draft, logits_target, draft_tokens, temperature, seed, offset,
                       nullptr, out_accept_len, out_tokens);
}

int spec_verify_noalloc(int batch, int gamma, int vocab, int dtype, void* hip_stream,
                        const void* logits_draft, const void* logits_target,
                        const int32_t* draft_tokens, const float* temperature, uint64_t seed,
                        uint64_t offset, int32_t* out_accept_len, int32_t* out_tokens) {
    const Shape shape{batch, gamma, vocab, dtype};
    Geometry geo;
    if (!shape_valid(shape) || !compute_geometry(shape, &geo))
        return SPEC_EINVAL;
    if (batch == 0)
        return SPEC_OK;
    if (!verify_args_valid(shape, logits_draft, logits_target, draft_tokens, temperature,
                           out_accept_len, out_tokens))
        return SPEC_EINVAL;
    if (layout_workspace(shape, geo, false, nullptr, nullptr) > kScratchBytes)
        return SPEC_ESCRATCH;
    void* base = nullptr;
    const int rc = scratch_address(&base);
    if (rc != SPEC_OK)
        return rc;
    Workspace ws;
    layout_workspace(shape, geo, false, static_cast<char*>(base), &ws);
    return verify_launch(shape, geo, ws, static_cast<hipStream_t>(hip_stream), logits_draft,
                         logits_target, draft_tokens, temperature, seed, offset, nullptr,
                         out_accept_len, out_tokens, LaunchEvents{}, LaunchEvents{},
                         LaunchEvents{});
}

int spec_verify_offset_ptr(spec_verify_ctx* ctx, const void* logits_draft,
                           const void* logits_target, const int32_t* draft_tokens,
                           const float* temperature, uint64_t seed, const uint64_t* offset_dev,
                           int32_t* out_accept_len, int32_t* out_tokens) {
    if (!offset_dev || !aligned(offset_dev, 8))
        return SPEC_EINVAL;
    return verify_impl(ctx, logits_draft, logits_target, draft_tokens, temperature, seed, 0,
                       offset_dev, out_accept_len, out_tokens);
}

int spec_accept_logprobs(spec_verify_ctx* ctx, const float* logprobs, uint64_t seed,
                         uint64_t offset, int32_t* out_accept_len) {
    if (!ctx)
        return SPEC_EINVAL;
    const Shape& s = ctx->shape;
    if (s.batch == 0)
        return SPEC_OK;
    if (!out_accept_len || (s.gamma > 0 && !logprobs))
        return SPEC_EINVAL;
    if ((logprobs && !aligned(logprobs, 8)) || !aligned(out_accept_len, 4))
        return SPEC_EINVAL;
    if (launch_accept_scalar(s.batch, s.gamma, logprobs, seed, offset, out_accept_len,
                             ctx->stream) != hipSuccess)
        return SPEC_EHIP;
    return SPEC_OK;
}

int spec_verify_outcomes(spec_verify_ctx* ctx, const void* logits_draft,
                         const void* logits_target, const int32_t* draft_tokens, int top_f,
                         int32_t* out_tokens, float* out_probs, float* out_pk, float* out_mass) {
    if (!ctx)
        return SPEC_EINVAL;
    const Shape& s = ctx->shape;
    if (top_f < 1 || top_f > SPEC_OUTCOME_MAX_F)
        return SPEC_EINVAL;
    if (s.batch == 0)
        return SPEC_OK;
    const size_t esz = s.dtype == SPEC_BF16 ? 2 : 4;
    if (!logits_target || !out_tokens || !out_probs || !out_pk)
        return SPEC_EINVAL;
    if (s.gamma > 0 && (!logits_draft || !draft_tokens))
        return SPEC_EINVAL;
    if (!aligned(logits_target, esz) || (logits_draft && !aligned(logits_draft, esz)) ||
        !aligned(out_tokens, 4) || !aligned(out_probs, 4) || !aligned(out_pk, 4) ||
        (out_mass && !aligned(out_mass, 4)) || (draft_tokens && !aligned(draft_tokens, 4)))
        return SPEC_EINVAL;
    if (!ctx->have_verified)
        return SPEC_ESTATE;
    if (s.gamma == 0)
        logits_draft = logits_target;
    const bool vec = (s.vocab % group_width(s.dtype)) == 0 && aligned(logits_target, 16) &&
                     aligned(logits_draft, 16);
    if (launch_outcomes(s, vec, ctx->geo.nsplit_outcome, top_f, logits_draft, logits_target,
                        draft_tokens, ctx->ws.seq, ctx->ws.rn, ctx->ws.lse, ctx->ws.gathered,
                        ctx->ws.outcome,
                        out_tokens, out_probs, out_pk, out_mass, ctx->stream) != hipSuccess)
        return SPEC_EHIP;
    return SPEC_OK;
}

int spec_verify_copy_lse(spec_verify_ctx* ctx, double* out_lse) {
    if (!ctx || !out_lse)
        return SPEC_EINVAL;
    if (!ctx->have_verified)
        return SPEC_ESTATE;
    const size_t n = static_cast<size_t>(ctx->shape.batch) * (2 * ctx->shape.gamma + 1);
    if (n == 0)
        return SPEC_OK;
    if (hipMemcpyAsync(out_lse, ctx->ws.lse, n * sizeof(double), hipMemcpyDeviceToDevice,
                       ctx->stream) != hipSuccess)
        return SPEC_EHIP;
    return SPEC_OK;
}

int spec_verify_philox_words(spec_verify_ctx* ctx, uint64_t seed, uint64_t offset,
                             uint32_t* out_words) {
    if (!ctx || !out_words || !aligned(out_words, 16))
        return SPEC_EINVAL;
    if (launch_philox_words(ctx->shape.batch, ctx->shape.gamma, seed, offset, out_words,
                            ctx->stream) != hipSuccess)
        return SPEC_EHIP;
    return SPEC_OK;
}

int spec_verify_enable_timing(spec_verify_ctx* ctx, int max_calls) {
    if (!ctx || max_calls < 0)
        return SPEC_EINVAL;
    for (hipEvent_t e : ctx->events)
        (void)hipEventDestroy(e);
    ctx->events.clear();
    ctx->timing_slots = 0;
    ctx->timing_count = 0;
    if (max_calls == 0)
        return SPEC_OK;
    ctx->events.resize(static_cast<size_t>(max_calls) * 6, nullptr);
    for (auto& e : ctx->events) {
        if (hipEventCreate(&e) != hipSuccess) {
            for (hipEvent_t x : ctx->events)
                if (x)
                    (void)hipEventDestroy(x);
            ctx->events.clear();
            return SPEC_EHIP;
        }
    }
    ctx->timing_slots = max_calls;
    return SPEC_OK;
}

int spec_verify_read_timing(spec_verify_ctx* ctx, float* out_ms, int max_calls) {
    if (!ctx || (max_calls > 0 && !out_ms))
        return SPEC_EINVAL;
    if (ctx->timing_slots == 0)
        return SPEC_ESTATE;
    const int recorded = std::min(ctx->timing_count, ctx->timing_slots);
    const int first = ctx->timing_count - recorded;
    int written = 0;
    for (int n = 0; n < recorded && written < max_calls; ++n) {
        hipEvent_t* ev = &ctx->events[static_cast<size_t>((first + n) % ctx->timing_slots) * 6];
        if (hipEventSynchronize(ev[5]) != hipSuccess)
            return SPEC_EHIP;
        for (int kk = 0; kk < 3; ++kk) {
            // the accept step runs inside the draw on the tile path: 0 here
            float ms = 0.0f;
            if ((kk != 1 || ctx->geo.nsplit_residual == 0) &&
                hipEventElapsedTime(&ms, ev[2 * kk], ev[2 * kk + 1]) != hipSuccess)
                return SPEC_EHIP;
            out_ms[written * 3 + kk] = ms;
        }
        ++written;
    }
    ctx->timing_count = 0;
    return written;
}

int spec_verify_get_geometry(spec_verify_ctx* ctx, int* out) {
    if (!ctx || !out)
        return SPEC_EINVAL;
    out[0] = ctx->geo.nsplit_rows;
    out[1] = ctx->geo.nsplit_residual;
    out[2] = kBlock;
    return SPEC_OK;
}

int spec_verify_destroy(spec_verify_ctx* ctx) {
    if (!ctx)
        return SPEC_EINVAL;
    int rc = SPEC_OK;
    if (hipStreamSynchronize(ctx->stream) != hipSuccess)
        rc = SPEC_EHIP;
    for (hipEvent_t e : ctx->events)
        (void)hipEventDestroy(e);
    if (ctx->ws_base && hipFree(ctx->ws_base) != hipSuccess)
        rc = SPEC_EHIP;
    delete ctx;
    return rc;
}

}  // extern "C"
