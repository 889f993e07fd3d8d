/*
 * spec_verify.h -- C ABI of the batched speculative-sampling verification
 * library for AMD Instinct MI355X (gfx950).
 *
 * The operation (sources: the pages' titles and sections):
 *   Given draft logits [B, G, V], target logits [B, G+1, V], draft tokens
 *   [B, G] and a temperature per sequence, decide on the device how many of
 *   the G draft tokens each sequence keeps and which extra token follows them,
 *   with no host round trip (FlashSpec technical summary, Problem statement
 *   item 1: host-side verification forces a device-to-host sync per decoding
 *   step; Methodology section 1: verification entirely on the device, two
 *   log-probability scalars per candidate token, log-space arithmetic,
 *   temperature applied before the log-softmax). The result is the
 *   "verification outcome" -- accepted count plus one token -- that the
 *   Speculative Speculative Decoding summary (section 2, central concept,
 *   item 1) consumes; the extra token comes from the residual distribution at
 *   the first rejection, or is the bonus token from the target when every
 *   draft token is kept (same summary, section 2, Saguaro challenge 2).
 *   The accept rule u < min(1, p/q) and the residual norm(max(0, p - q)) are
 *   those of standard speculative sampling (Leviathan, Kalman and Matias,
 *   ICML 2023), which keeps the target's output distribution exactly, as the
 *   FlashSpec summary requires (Methodology intro; Theorem 1).
 *
 * Precise definition, per sequence b with T = temperature[b], t_i = draft
 * token i:
 *   x = fl32(z * fl32(1/T)) for every logit z (binary32, round to nearest);
 *   lse_q[i] = log sum_v exp(xq[i][v]) over draft row i (i < G);
 *   lse_p[i] = log sum_v exp(xp[i][v]) over target row i (i <= G);
 *   position i < G is accepted iff log(u_acc(b,i)) < (xp[i][t_i] - lse_p[i])
 *                                                  - (xq[i][t_i] - lse_q[i]);
 *   k = first rejected position, or G;
 *   if k < G the extra token is drawn from r_v = max(0, p_k(v) - q_k(v)),
 *   if k == G from r_v = p_G(v), by inversion: the first index v (in
 *   vocabulary order) whose inclusive prefix sum of r exceeds u_res(b,k) * S,
 *   S = sum_v r_v; an empty residual (S == 0) draws from p_k instead.
 *   T == 0 is greedy: position i is accepted iff t_i == argmax_v z_p[i][v]
 *   (raw logits, lowest index on ties) and the extra token is argmax z_p[k].
 *   Uniforms: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11), key
 *   (lo32(seed), hi32(seed)), counter (i, b, lo32(offset), hi32(offset)) for
 *   i = 0..G; u_acc(b,i) = (word0 >> 8) * 2^-24, u_res(b,i) = (word1 >> 8) *
 *   2^-24. Outputs are a pure function of the inputs and (seed, offset); the
 *   caller advances offset by one per call.
 *
 * Layouts: every array is dense, row-major, with the vocabulary innermost.
 * Logits are binary32 (SPEC_F32) or bfloat16 (SPEC_BF16); pointers must be
 * aligned to the element size. Tokens and lengths are int32. Every pointer
 * passed to spec_verify / spec_accept_logprobs / the test hooks is a DEVICE
 * pointer owned by the caller, and must stay valid until the work queued on
 * the context's stream has completed. The library owns only its workspace.
 *
 * Asynchrony: calls enqueue kernels on the context's stream and return
 * without synchronising the host. One context per stream; a context is not
 * thread-safe and two calls on one context must not run concurrently.
 *
 * Errors: host-detectable problems (NULL context or pointer, bad shape or
 * dtype, misaligned pointer) return a negative status before any launch. A
 * failed launch returns SPEC_EHIP. Bad DATA is reported per sequence without
 * a host sync: a temperature that is NaN, negative or +inf, or whose
 * reciprocal overflows, a draft token outside [0, V), or a row the sequence
 * uses that has no finite logit gives out_accept_len[b] = -1 and
 * out_tokens[b, :] = -1. Logits equal to +inf or NaN are a precondition
 * violation: the result is unspecified but no out-of-bounds access happens.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct spec_verify_ctx spec_verify_ctx;

enum spec_dtype { SPEC_F32 = 0, SPEC_BF16 = 1 };

enum spec_status {
    SPEC_OK = 0,
    SPEC_EINVAL = -1, /* bad argument: NULL, shape, dtype, alignment        */
    SPEC_EHIP = -2,   /* a HIP runtime call or kernel launch failed          */
    SPEC_ENOMEM = -3, /* workspace allocation failed                         */
    SPEC_ESTATE = -4, /* context in the wrong state for this call           */
    SPEC_ESCRATCH = -5 /* the shape's workspace exceeds the fixed scratch array
                          of spec_verify_noalloc                             */
};

/*
 * Create a context for batches of `batch` sequences, `gamma` >= 0 draft
 * tokens each and a vocabulary of `vocab` >= 1 entries, logits of `dtype`,
 * launching on `hip_stream` (a hipStream_t; NULL = the null stream).
 * Allocates the device workspace (a few MB at the largest shapes) and
 * zeroes its counters. The shape is fixed for the context's lifetime.
 * batch * (2*gamma+1) and vocab must each be below 2^31.
 * Returns SPEC_OK and *out_ctx, or a negative status and *out_ctx = NULL.
 *
 * The launch geometry is chosen here from the shape. For tuning, these
 * environment variables, read once by this call, override it (results do not
 * depend on them, except that the arithmetic order of the split merges
 * follows the split count):
 *   SPEC_VERIFY_ROW_SPLIT       vocabulary splits per row of the row kernel
 *                               (> 0; capped at 64 and at the row's batches)
 *   SPEC_VERIFY_ROW_UNROLL      16-byte groups in flight per thread: 2, 4, 8
 *   SPEC_VERIFY_ROW_NT          0: ordinary instead of non-temporal loads
 *   SPEC_VERIFY_RESIDUAL_FUSED  0/1: one workgroup per sequence for the draw
 *                               (default from B = 128)
 *   SPEC_VERIFY_RESIDUAL_SPLIT  vocabulary splits of the tile-sum kernel (> 0;
 *                               selects the two-kernel draw)
 *   SPEC_VERIFY_RESIDUAL_UNROLL tiles per batch in that kernel: 2 or 4
 *   SPEC_VERIFY_OUTCOME_SPLIT   vocabulary splits of spec_verify_outcomes
 */
int spec_verify_init(int batch, int gamma, int vocab, int dtype, void *hip_stream,
                     spec_verify_ctx **out_ctx);

/* Move later launches of this context to another stream (hipStream_t). */
int spec_verify_set_stream(spec_verify_ctx *ctx, void *hip_stream);

/*
 * The full verification (definition above). Device pointers:
 *   logits_draft   [B, G, V]    dtype; may be NULL iff G == 0
 *   logits_target  [B, G+1, V]  dtype
 *   draft_tokens   [B, G]       int32; may be NULL iff G == 0
 *   temperature    [B]          float32; 0 selects greedy verification
 *   out_accept_len [B]          int32: k, or -1 for a rejected sequence
 *   out_tokens     [B, G+1]     int32: tokens[0..k) = draft, tokens[k] =
 *                               the extra token, the rest -1
 * Enqueues its kernels on the context's stream and returns: row
 * normalisers; gather, accept and first rejection; the residual or bonus
 * draw. From B = 128 these are three kernels (the draw one workgroup per
 * sequence); below, the accept step runs inside the draw's tile-sum kernel,
 * followed by a locate kernel.
 */
int spec_verify(spec_verify_ctx *ctx, const void *logits_draft,
                const void *logits_target, const int32_t *draft_tokens,
                const float *temperature, uint64_t seed, uint64_t offset,
                int32_t *out_accept_len, int32_t *out_tokens);

/*
 * spec_verify with the Philox offset read on the device from *offset_dev
 * (one uint64 word, device memory, 8-byte aligned, owned by the caller) when
 * the accept kernel runs, instead of passed by value. A call recorded into a
 * HIP graph then draws fresh uniforms on every replay if the caller advances
 * the word between replays (for instance with a one-element add recorded in
 * the same graph); every other argument and result is as for spec_verify,
 * which this equals bit for bit when *offset_dev holds the same offset.
 * Returns SPEC_EINVAL for a NULL or misaligned offset_dev.
 */
int spec_verify_offset_ptr(spec_verify_ctx *ctx, const void *logits_draft,
                           const void *logits_target, const int32_t *draft_tokens,
                           const float *temperature, uint64_t seed,
                           const uint64_t *offset_dev, int32_t *out_accept_len,
                           int32_t *out_tokens);

/* Size of the fixed device scratch array of spec_verify_noalloc: 16 MiB. */
#define SPEC_VERIFY_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * spec_verify without a context: same arguments, definition, launch geometry
 * (computed per call on the host from the shape, as spec_verify_init does)
 * and kernels, so it equals spec_verify bit for bit. Its workspace is a fixed
 * file-scope device array of SPEC_VERIFY_NOALLOC_SCRATCH_BYTES bytes instead
 * of an allocation; every GPU the library runs on holds its own copy until
 * the process ends. The call allocates and frees nothing (no hipMalloc,
 * hipFree or allocating library routine); on its first call on a device it
 * looks up that device's copy with hipGetSymbolAddress and keeps the address.
 * Returns SPEC_ESCRATCH, before any launch, when the shape needs more
 * workspace than the array holds (B = 256, G = 8, V = 152064 needs about
 * 0.5 MiB), and the statuses of spec_verify otherwise. Calls on one device
 * share the array, which keeps the last call's contents (every entry a call
 * reads is written by that call first): calls that overlap in time on one
 * device (on different streams, or from several host threads) race and give
 * wrong results. hip_stream is a hipStream_t (NULL = the null stream).
 */
int spec_verify_noalloc(int batch, int gamma, int vocab, int dtype, void *hip_stream,
                        const void *logits_draft, const void *logits_target,
                        const int32_t *draft_tokens, const float *temperature,
                        uint64_t seed, uint64_t offset, int32_t *out_accept_len,
                        int32_t *out_tokens);

/*
 * Scalar-only mode: reads only the gathered log-probability pairs, O(B*G)
 * bytes, nothing of size V (FlashSpec summary, Methodology section 1,
 * mechanism and complexity bullets). Device pointers:
 *   logprobs       [B, G, 2] float32: [..., 0] = log q (draft),
 *                  [..., 1] = log p (target), temperature already applied
 *   out_accept_len [B] int32
 * Same counters and accept test as spec_verify: position i is accepted iff
 * log(u_acc(b,i)) < (double)lp - (double)lq (IEEE: NaN rejects). No extra
 * token is drawn (there is no distribution to draw from) and no greedy mode.
 */
int spec_accept_logprobs(spec_verify_ctx *ctx, const float *logprobs, uint64_t seed,
                         uint64_t offset, int32_t *out_accept_len);

/* Longest top-F list of spec_verify_outcomes. */
#define SPEC_OUTCOME_MAX_F 64

/*
 * The law of the last verification's outcome given its drafts: the pair
 * (accepted count k, extra token) that speculative speculative decoding
 * predicts and keys its speculation cache on, spending the cache on likely
 * lengths and, per length, on the top-F tokens of the residual distribution
 * (Speculative Speculative Decoding summary, section 2: central concept,
 * Saguaro challenges 1 and 2). For every sequence b and length i in [0, G]:
 *   out_pk[b,i]   = P(k = i | drafts): prod_{j<i} beta_j * (1 - beta_i) for
 *                   i < G and prod_{j<G} beta_j for i = G, with beta_j =
 *                   min(1, p_j(t_j) / q_j(t_j)) from the accept test's
 *                   log-probabilities (0 when their difference is NaN);
 *   out_tokens[b,i,:F], out_probs[b,i,:F] = the F most likely extra tokens
 *                   at length i and their probabilities, largest first, the
 *                   lower index first among equal values: the residual
 *                   max(0, p_i - q_i) / S_i for i < G, p_G for i = G, p_i when
 *                   S_i = 0; token -1 and probability 0 past the vocabulary;
 *   out_mass[b,i] = S_i = sum_v max(0, p_i - q_i) (the total-variation
 *                   distance of p_i and q_i) for i < G, 1 for i = G.
 * Greedy sequences (T == 0) have a deterministic outcome: lists by raw target
 * logit with probabilities 1, 0, ..., P(k = i) in {0, 1}, mass 0. Sentinel
 * sequences get tokens -1 and zeros. Probabilities use the row normalisers
 * and the arithmetic of the verification (binary32 exp2 of the scaled
 * logits), so they carry a relative error of a few 1e-6.
 *
 * Must follow a spec_verify call on the same context with the same logits,
 * draft tokens and temperatures: it reuses that call's row normalisers,
 * gathered logits and per-sequence state (SPEC_ESTATE if there was none).
 * Reads the logits once more. Device pointers:
 *   logits_draft [B, G, V], logits_target [B, G+1, V], draft_tokens [B, G]
 *   (as given to spec_verify; draft pointers may be NULL iff G == 0);
 *   out_tokens [B, G+1, F] int32, out_probs [B, G+1, F] float32,
 *   out_pk [B, G+1] float32, out_mass [B, G+1] float32 (may be NULL);
 *   1 <= top_f <= SPEC_OUTCOME_MAX_F.
 */
int spec_verify_outcomes(spec_verify_ctx *ctx, const void *logits_draft,
                         const void *logits_target, const int32_t *draft_tokens, int top_f,
                         int32_t *out_tokens, float *out_probs, float *out_pk,
                         float *out_mass);

/* Largest number of lengths spec_outcome_fanout takes. */
#define SPEC_FANOUT_MAX_LENGTHS 256

/*
 * Speculation-cache budget per length: how many of each length's listed
 * tokens to speculate on with a budget of `budget` cache entries per sequence
 * (Speculative Speculative Decoding summary, section 2, Saguaro challenge 1:
 * the budget goes unevenly to the lengths, more to likely ones and fewer to
 * unlikely ones, so that a fixed budget hits the cache as often as it can; the
 * page names a geometric allocation without a formula). An entry is a pair
 * (length i, the j-th token of length i's list), worth
 *   v(i, j) = pk[b,i] * probs[b,i,j]   (product in binary64, exact; 0 when
 *                                       negative or NaN),
 * the probability that the verification outcome is that pair. Entries are
 * placed one at a time, each on the length whose next unused list entry is
 * worth the most (the lower length on equal worth), until `budget` are placed
 * or every list is used up. Each length gets a prefix of its list:
 *   out_n[b,i]  = entries placed at length i (the first out_n[b,i] tokens of
 *                 its list), sum_i out_n[b,i] = min(budget, lengths * top_f);
 *   out_hit[b]  = the sum of the placed worths (binary64, summed in an order
 *                 of the kernel's choosing, the same on every call): the
 *                 expected cache hit rate.
 * For lists that are non-increasing, as spec_verify_outcomes writes them, the
 * placed entries are the `budget` most valuable pairs, which maximises the
 * hit rate; the page's geometric allocation is the case of pk geometric in i
 * (a fixed acceptance rate alpha: pk[i] = alpha^i (1 - alpha), alpha^G at G).
 * Device pointers, float32 / int32 / float64, launched on `hip_stream` (a
 * hipStream_t, NULL = the null stream), asynchronous:
 *   pk [B, lengths], probs [B, lengths, top_f] (spec_verify_outcomes' out_pk
 *   and out_probs, lengths = G + 1), out_n [B, lengths], out_hit [B] (may be
 *   NULL). 1 <= lengths <= SPEC_FANOUT_MAX_LENGTHS, 1 <= top_f <=
 *   SPEC_OUTCOME_MAX_F, budget >= 0, batch >= 0; SPEC_EINVAL otherwise (or
 *   for NULL or misaligned pointers), SPEC_EHIP if the launch fails.
 */
int spec_outcome_fanout(int batch, int lengths, int top_f, const float *pk, const float *probs,
                        int budget, int32_t *out_n, double *out_hit, void *hip_stream);

/*
 * Test hook: copy the row log-normalisers of the last spec_verify call into
 * out_lse [B, 2G+1] float64 (device): draft rows 0..G-1, then target rows
 * 0..G. Rows not computed (greedy or rejected sequences) are NaN. Enqueued
 * on the context's stream.
 */
int spec_verify_copy_lse(spec_verify_ctx *ctx, double *out_lse);

/*
 * Test hook: the raw Philox words the kernels use, out_words [B, G+1, 4]
 * uint32 (device), for (seed, offset). Enqueued on the context's stream.
 */
int spec_verify_philox_words(spec_verify_ctx *ctx, uint64_t seed, uint64_t offset,
                             uint32_t *out_words);

/*
 * Per-kernel timing. spec_verify_enable_timing(ctx, n) makes each following
 * spec_verify call attach a start and a stop HIP event to the dispatches of
 * its three steps (hipExtLaunchKernel; the split draw's pair of kernels is
 * timed from the first's start to the second's stop), on the context's
 * stream, into a ring of n slots (n = 0 turns it off). The events time the
 * kernels alone and add no packet of their own between them. Below B = 128
 * the draw's tile kernel runs the accept step itself, so that step's
 * duration reads 0 and the draw's includes it.
 * spec_verify_read_timing waits for the recorded calls, writes up to
 * max_calls rows of three durations in milliseconds (row normalisers,
 * accept, residual) into out_ms (HOST memory, [max_calls, 3]), returns the
 * number of rows written (or a negative status) and empties the ring.
 */
int spec_verify_enable_timing(spec_verify_ctx *ctx, int max_calls);
int spec_verify_read_timing(spec_verify_ctx *ctx, float *out_ms, int max_calls);

/* Launch geometry chosen at init: vocabulary splits of the row-normaliser and
 * residual kernels (0 for the residual: one workgroup per sequence, the tile
 * sums kept in LDS), and threads per workgroup of the vocabulary kernels.
 * Host memory out[3]. */
int spec_verify_get_geometry(spec_verify_ctx *ctx, int *out);

/* Free the workspace and the context (waits for the context's stream). */
int spec_verify_destroy(spec_verify_ctx *ctx);

/*
 * Measurement utility (not part of the verification): a read-only streaming
 * probe of HBM, the practical ceiling the streaming kernels are compared with
 * beside the vendor peak. Reads `bytes` (a multiple of 16) of the device
 * buffer `buf` (16-byte aligned) with 16-byte non-temporal loads, one
 * contiguous run per workgroup of 256 threads (`blocks` of them; the row
 * kernel's access pattern), and writes one word per workgroup into
 * the device array sink[blocks] (4-byte aligned) so the loads are kept.
 * Enqueued on hip_stream (a hipStream_t; NULL = the null stream).
 */
int spec_hbm_read_probe(const void *buf, uint64_t bytes, uint32_t *sink, int blocks,
                        void *hip_stream);

/* A static description of a status code. */
const char *spec_verify_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
