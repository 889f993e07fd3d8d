// The C ABI (include/spec_verify.h): context, workspace, argument checks and
// the launch sequence row-normaliser -> accept -> residual on one stream.
// Nothing here synchronises the host except spec_verify_read_timing and
// spec_verify_destroy.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <new>
#include <vector>

#include "launch.hpp"
#include "outcome.hpp"
#include "spec_verify.h"

using namespace specv;

struct spec_verify_ctx {
    Shape shape{};
    hipStream_t stream = nullptr;
    int device = 0;
    int nsplit_rows = 1;      // vocabulary splits of the row-normaliser kernel
    int row_unroll = 8;       // 16-byte groups in flight per thread in that kernel
    bool row_nontemporal = true;
    int nsplit_residual = 1;  // vocabulary splits of the residual kernel
    int residual_unroll = 4;  // tiles per batch per wavefront in that kernel
    int nsplit_outcome = 1;   // vocabulary splits of the outcome kernel

    void* ws = nullptr;
    Partial* part = nullptr;
    float* gathered = nullptr;
    RowNorm* rn = nullptr;
    double* lse = nullptr;
    SeqState* seq = nullptr;
    float* tile_sums = nullptr;
    OutcomeWork outcome{};
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
constexpr long kOutcomeTargetBlocks = 2048;
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

}  // namespace

extern "C" {

const char* spec_verify_strerror(int code) {
    switch (code) {
    case SPEC_OK: return "ok";
    case SPEC_EINVAL: return "invalid argument";
    case SPEC_EHIP: return "HIP runtime error";
    case SPEC_ENOMEM: return "out of device memory";
    case SPEC_ESTATE: return "context in the wrong state for this call";
    default: return "unknown status";
    }
}

int spec_verify_init(int batch, int gamma, int vocab, int dtype, void* hip_stream,
                     spec_verify_ctx** out_ctx) {
    if (!out_ctx)
        return SPEC_EINVAL;
    *out_ctx = nullptr;
    if (batch < 0 || gamma < 0 || vocab < 1 || (dtype != SPEC_F32 && dtype != SPEC_BF16))
        return SPEC_EINVAL;
    const long rows = static_cast<long>(batch) * (2L * gamma + 1);
    if (rows >= (1L << 31) || static_cast<long>(batch) * (gamma + 1) >= (1L << 31))
        return SPEC_EINVAL;

    spec_verify_ctx* ctx = new (std::nothrow) spec_verify_ctx();
    if (!ctx)
        return SPEC_ENOMEM;
    ctx->shape = Shape{batch, gamma, vocab, dtype};
    ctx->stream = static_cast<hipStream_t>(hip_stream);
    if (hipGetDevice(&ctx->device) != hipSuccess) {
        delete ctx;
        return SPEC_EHIP;
    }
    ctx->nsplit_rows = choose_split(rows, vocab, dtype, kRowTargetBlocks, 4L * kBlock);
    ctx->nsplit_residual = choose_split(batch, vocab, dtype, kResidualTargetBlocks, 16L * 64);
    const long pairs = static_cast<long>(batch) * (gamma + 1);
    ctx->nsplit_outcome = std::min(kOutcomeMaxSplit,
                                   choose_split(pairs, vocab, dtype, kOutcomeTargetBlocks, 16L * 64));
    const int oo = env_int("SPEC_VERIFY_OUTCOME_SPLIT", 0);
    if (oo > 0)
        ctx->nsplit_outcome = std::min(oo, kOutcomeMaxSplit);
    const int o1 = env_int("SPEC_VERIFY_ROW_SPLIT", 0), o3 = env_int("SPEC_VERIFY_RESIDUAL_SPLIT", 0);
    if (o1 > 0)
        ctx->nsplit_rows = std::min(o1, kMaxSplit);
    if (o3 > 0)
        ctx->nsplit_residual = std::min(o3, kMaxSplit);
    const int ou = env_int("SPEC_VERIFY_ROW_UNROLL", 0);
    if (ou == 2 || ou == 4 || ou == 8)
        ctx->row_unroll = ou;
    // Row splits are whole batch strides (unroll x kBlock groups): more splits
    // than strides would only add empty splits for the accept kernel to merge.
    // Unless the rows alone are too few to give every CU a few workgroups, a
    // split also keeps about three batches per thread, so that a thread's
    // loads overlap each other and the block's closing reduction is paid for
    // by more than one batch (at B = 64, V = 128256: 2 splits instead of 8,
    // 57.1 -> 51.6 us per call).
    {
        const long stride = static_cast<long>(ctx->row_unroll) * kBlock;
        const long strides = std::max(1L, (vocab / group_width(dtype) + stride - 1) / stride);
        long n = std::min<long>(ctx->nsplit_rows, strides);
        if (o1 <= 0) {
            const long fill = rows > 0 ? (kRowFillBlocks + rows - 1) / rows : 1;
            n = std::min(n, std::max(fill, std::max(1L, strides / 3)));
        }
        ctx->nsplit_rows = static_cast<int>(n);
    }
    ctx->row_nontemporal = env_int("SPEC_VERIFY_ROW_NT", ctx->row_nontemporal ? 1 : 0) != 0;
    const int ru = env_int("SPEC_VERIFY_RESIDUAL_UNROLL", 0);
    if (ru == 2 || ru == 4)
        ctx->residual_unroll = ru;
    // With at least half as many sequences as CUs, one workgroup per sequence
    // (the fused residual kernel) fills the GPU by itself.
    const bool fused_fits = residual_tiles_per_row(vocab) <= residual_fused_max_tiles();
    int fused = batch >= kResidualFusedMinBatch && fused_fits ? 1 : 0;
    fused = env_int("SPEC_VERIFY_RESIDUAL_FUSED", fused);
    if (fused && fused_fits && o3 <= 0)
        ctx->nsplit_residual = 0;
    // A dispatch holds fewer than 2^32 work-items.
    const long long limit = 1LL << 32;
    if (static_cast<long long>(rows) * ctx->nsplit_rows * kBlock >= limit ||
        static_cast<long long>(batch) * std::max(ctx->nsplit_residual, 1) * kBlock >= limit ||
        static_cast<long long>(pairs) * ctx->nsplit_outcome * kBlock >= limit) {
        delete ctx;
        return SPEC_EINVAL;
    }

    // Workspace: one allocation, 256-byte aligned sub-arrays.
    const size_t n_part = static_cast<size_t>(rows) * ctx->nsplit_rows;
    size_t off = 0;
    const size_t o_part = off; off = align_up(off + n_part * sizeof(Partial), 256);
    const size_t o_rn = off;   off = align_up(off + rows * sizeof(RowNorm), 256);
    const size_t o_ga = off;   off = align_up(off + rows * sizeof(float), 256);
    const size_t o_lse = off;  off = align_up(off + rows * sizeof(double), 256);
    const size_t o_seq = off;  off = align_up(off + static_cast<size_t>(batch) * sizeof(SeqState), 256);
    const size_t o_ts = off;   off = align_up(off + static_cast<size_t>(batch) * residual_tiles_per_row(vocab) * sizeof(float), 256);
    const size_t n_oc = static_cast<size_t>(pairs) * ctx->nsplit_outcome;
    const size_t o_oc = off;   off = align_up(off + n_oc * kOutcomeMaxF * sizeof(Cand), 256);
    const size_t o_os = off;   off = align_up(off + n_oc * sizeof(double), 256);
    const size_t total = std::max<size_t>(off, 256);
    if (hipMalloc(&ctx->ws, total) != hipSuccess) {
        delete ctx;
        return SPEC_ENOMEM;
    }
    char* base = static_cast<char*>(ctx->ws);
    ctx->part = reinterpret_cast<Partial*>(base + o_part);
    ctx->rn = reinterpret_cast<RowNorm*>(base + o_rn);
    ctx->gathered = reinterpret_cast<float*>(base + o_ga);
    ctx->lse = reinterpret_cast<double*>(base + o_lse);
    ctx->seq = reinterpret_cast<SeqState*>(base + o_seq);
    ctx->tile_sums = reinterpret_cast<float*>(base + o_ts);
    ctx->outcome.cand = reinterpret_cast<Cand*>(base + o_oc);
    ctx->outcome.sums = reinterpret_cast<double*>(base + o_os);
    // Defined contents before the first call (every entry is rewritten by it).
    if (hipMemset(ctx->ws, 0, total) != hipSuccess) {
        (void)hipFree(ctx->ws);
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

// The verification call; the Philox offset is `offset`, or the device word
// *offset_dev when that is non-null.
int verify_impl(spec_verify_ctx* ctx, const void* logits_draft, const void* logits_target,
                const int32_t* draft_tokens, const float* temperature, uint64_t seed,
                uint64_t offset, const uint64_t* offset_dev, int32_t* out_accept_len,
                int32_t* out_tokens) {
    if (!ctx)
        return SPEC_EINVAL;
    const Shape& s = ctx->shape;
    if (s.batch == 0)
        return SPEC_OK;
    const size_t esz = s.dtype == SPEC_BF16 ? 2 : 4;
    if (!logits_target || !temperature || !out_accept_len || !out_tokens)
        return SPEC_EINVAL;
    if (s.gamma > 0 && (!logits_draft || !draft_tokens))
        return SPEC_EINVAL;
    if (!aligned(logits_target, esz) || (logits_draft && !aligned(logits_draft, esz)) ||
        !aligned(temperature, 4) || !aligned(out_accept_len, 4) || !aligned(out_tokens, 4) ||
        (draft_tokens && !aligned(draft_tokens, 4)))
        return SPEC_EINVAL;
    if (s.gamma == 0)
        logits_draft = logits_target;  // never read; keeps the kernels' pointers valid

    // 16-byte groups need every row start 16-byte aligned.
    const bool vec = (s.vocab % group_width(s.dtype)) == 0 && aligned(logits_target, 16) &&
                     aligned(logits_draft, 16);

    // Timing mode: each step's start and stop events ride on its kernels'
    // own dispatches, so they time the kernels alone.
    LaunchEvents ev_row, ev_acc, ev_res;
    if (ctx->timing_slots > 0) {
        hipEvent_t* ev = &ctx->events[static_cast<size_t>(ctx->timing_count % ctx->timing_slots) * 6];
        ++ctx->timing_count;
        ev_row = LaunchEvents{ev[0], ev[1]};
        ev_acc = LaunchEvents{ev[2], ev[3]};
        ev_res = LaunchEvents{ev[4], ev[5]};
    }
    hipStream_t st = ctx->stream;
    const RowTuning tu{ctx->nsplit_rows, ctx->row_unroll, ctx->row_nontemporal};
    if (launch_row_norm(s, vec, tu, logits_draft, logits_target, temperature, draft_tokens,
                        ctx->part, ctx->gathered, st, ev_row) != hipSuccess)
        return SPEC_EHIP;
    const AcceptArgs acc{draft_tokens, temperature, s.gamma, s.vocab, ctx->nsplit_rows, seed,
                         offset, offset_dev, ctx->part, ctx->gathered, ctx->rn, ctx->lse,
                         ctx->seq, out_accept_len, out_tokens};
    // On the tile path (small batches) the tile kernel runs the accept step
    // itself, which saves a launch; the fused draw needs the accept kernel.
    const bool fold = ctx->nsplit_residual > 0;
    if (!fold && launch_accept(s.batch, acc, st, ev_acc) != hipSuccess)
        return SPEC_EHIP;
    if (launch_residual(s, vec, ctx->nsplit_residual, ctx->residual_unroll, logits_draft,
                        logits_target, ctx->seq, ctx->tile_sums, out_tokens, fold ? &acc : nullptr,
                        st, ev_res) != hipSuccess)
        return SPEC_EHIP;
    ctx->have_verified = true;
    return SPEC_OK;
}

}  // namespace

extern "C" {

int spec_verify(spec_verify_ctx* ctx, const void* logits_draft, const void* logits_target,
                const int32_t* draft_tokens, const float* temperature, uint64_t seed,
                uint64_t offset, int32_t* out_accept_len, int32_t* out_tokens) {
    return verify_impl(ctx, logits_draft, logits_target, draft_tokens, temperature, seed, offset,
                       nullptr, out_accept_len, out_tokens);
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
    if (launch_outcomes(s, vec, ctx->nsplit_outcome, top_f, logits_draft, logits_target,
                        draft_tokens, ctx->seq, ctx->rn, ctx->lse, ctx->gathered, ctx->outcome,
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
    if (hipMemcpyAsync(out_lse, ctx->lse, n * sizeof(double), hipMemcpyDeviceToDevice,
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
            if ((kk != 1 || ctx->nsplit_residual == 0) &&
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
    out[0] = ctx->nsplit_rows;
    out[1] = ctx->nsplit_residual;
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
    if (ctx->ws && hipFree(ctx->ws) != hipSuccess)
        rc = SPEC_EHIP;
    delete ctx;
    return rc;
}

}  // extern "C"
