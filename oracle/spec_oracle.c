/*
 * spec_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded CPU reference for batched speculative-sampling
 * verification, written for readability, not speed. Only the test suite, the
 * package smoke check and the benchmark's CPU-baseline leg may load it. The
 * HIP library never links, calls or includes anything from this directory, and
 * this file includes nothing from the HIP library.
 *
 * Every floating-point step after the two fp32 roundings named in step 3 below
 * is done in IEEE double, with the obvious loop order. No blocking, no fusion.
 *
 * What is computed, per sequence b (sources are the pages' titles and sections):
 *   1. Temperature is applied to the logits BEFORE the log-softmax, and the test
 *      works in log space on two log-probability scalars per draft token, one
 *      from the draft model and one from the target
 *      (FlashSpec technical summary, Methodology section 1, "on-device
 *      verification kernel": mechanism and numerical-stability bullets; the
 *      "engineering rigour" bullet of its Significance section repeats the
 *      temperature-order lesson).
 *   2. The verification outcome is the number of accepted draft tokens plus
 *      one extra token: drawn from the residual distribution at the first
 *      rejected position, or the "bonus" token when all are accepted
 *      (Speculative Speculative Decoding summary, section 2: central concept
 *      item 1 names the outcome (#accepted, bonus token); Saguaro challenge 2
 *      names the residual distribution the bonus token is sampled from).
 *   3. The result must have exactly the target model's output distribution
 *      (FlashSpec summary, Methodology intro and Theorem 1 in Significance).
 *      The pages give no formulas for 1-3; the accept rule u < min(1, p/q) and
 *      the residual norm(max(0, p - q)) used here are the standard speculative
 *      sampling rule (Leviathan, Kalman and Matias, ICML 2023; Chen et al.
 *      2023), the rule that has the exactness property the pages claim.
 *
 * Readings taken where the pages are silent (each is stated again where used):
 *   R1 target position i scores draft token i; target position gamma is the bonus;
 *   R3 x = fl32(z * fl32(1/T)), one temperature per sequence for draft and target;
 *   R4 T == 0 is greedy: accept iff token == argmax of raw target logits (lowest
 *      index on ties); the extra token is that argmax; no uniforms are used;
 *   R5 uniforms are 24-bit in [0, 1), the accept test is a strict '<';
 *   R6 Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) with key
 *      (lo32(seed), hi32(seed)) and counter (i, b, lo32(offset), hi32(offset));
 *      word 0 gives the accept uniform of position i, word 1 the resample
 *      uniform used at the first rejected position (or at gamma for the bonus);
 *   R7 the residual CDF runs in vocabulary-index order; the token is the first
 *      index whose inclusive prefix sum exceeds u * S;
 *   R8 a residual with S <= 0 (impossible in exact arithmetic after a
 *      rejection) falls back to p at that position;
 *   R12 gamma == 0 means no draft rows; accept length 0 and a bonus draw;
 *   R13 -inf logits are allowed; +inf / NaN logits are a precondition violation;
 *   sentinel: a sequence whose temperature is NaN, negative, +inf or whose
 *      reciprocal overflows, or whose draft token lies outside [0, V), or one
 *      of whose rows has no finite logit, gets accept_len = -1 and tokens -1.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* binary32 expressions must be evaluated in binary32 for step 3 to hold */
#if !defined(FLT_EVAL_METHOD) || FLT_EVAL_METHOD != 0
#error "the oracle needs FLT_EVAL_METHOD == 0"
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* ---------------------------------------------------------------- inputs -- */

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static float bf16_bits_to_float(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Raw logit z at flat element index idx of a row-major array. */
static float raw_logit(const void *base, int dtype, size_t idx)
{
    if (dtype == ORACLE_BF16)
        return bf16_bits_to_float(((const uint16_t *)base)[idx]);
    return ((const float *)base)[idx];
}

/* ---------------------------------------------------- Philox4x32-10 -------- */

/*
 * Philox4x32 with 10 rounds, from its published definition (Salmon et al.,
 * SC'11, section on the Philox S-box): each round multiplies counter words 0
 * and 2 by two fixed 32-bit constants into 64-bit products, and the new
 * counter is (hi(c2*M1) ^ c1 ^ k0, lo(c2*M1), hi(c0*M0) ^ c3 ^ k1, lo(c0*M0)).
 * Between rounds the key is bumped by the two Weyl constants.
 */
void oracle_philox4x32_10(const uint32_t counter[4], const uint32_t key[2],
                          uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = counter[0], c1 = counter[1], c2 = counter[2], c3 = counter[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        uint64_t prod0 = (uint64_t)M0 * (uint64_t)c0;
        uint64_t prod1 = (uint64_t)M1 * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
        uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The four Philox words of block (b, i) for a given seed and offset (R6). */
void oracle_philox_words(uint64_t seed, uint64_t offset, int64_t b, int i,
                         uint32_t out[4])
{
    uint32_t key[2] = { (uint32_t)seed, (uint32_t)(seed >> 32) };
    uint32_t ctr[4] = { (uint32_t)i, (uint32_t)b,
                        (uint32_t)offset, (uint32_t)(offset >> 32) };
    oracle_philox4x32_10(ctr, key, out);
}

/* 24-bit uniform in [0, 1) from one 32-bit word (R5): top 24 bits times 2^-24. */
double oracle_uniform24(uint32_t word)
{
    return (double)(word >> 8) * (1.0 / 16777216.0);
}

/* ------------------------------------------------------- row reductions -- */

/* The temperature-scaled logit of R3: x = fl32(z * fl32(1/T)), one binary32
 * multiply rounded to nearest (the file is built with contraction off). */
static float scaled(float z, float inv_t)
{
    float x = z * inv_t;
    return x;
}

/*
 * Log-sum-exp of one row of scaled logits, two passes in double:
 * M = max_v x_v over finite entries, lse = M + log(sum_v exp(x_v - M)).
 * Returns -inf when the row has no finite entry.
 */
double oracle_row_lse(const void *row_base, int dtype, size_t row_elem0,
                      int vocab, float inv_t)
{
    double m = -INFINITY;
    for (int v = 0; v < vocab; ++v) {
        double x = scaled(raw_logit(row_base, dtype, row_elem0 + (size_t)v), inv_t);
        if (x > m)
            m = x;
    }
    if (!(m > -INFINITY))
        return -INFINITY;
    double s = 0.0;
    for (int v = 0; v < vocab; ++v) {
        double x = scaled(raw_logit(row_base, dtype, row_elem0 + (size_t)v), inv_t);
        s += exp(x - m);
    }
    return m + log(s);
}

/* Index of the largest raw logit of a row, lowest index on ties (R4); -1 when
 * the row has no finite entry. */
int oracle_row_argmax(const void *row_base, int dtype, size_t row_elem0, int vocab)
{
    int best = -1;
    float best_z = -INFINITY;
    for (int v = 0; v < vocab; ++v) {
        float z = raw_logit(row_base, dtype, row_elem0 + (size_t)v);
        if (z > best_z) {
            best_z = z;
            best = v;
        }
    }
    return best;
}

/*
 * Inverse-CDF draw from weights r_v >= 0 (R7): S = sum r in index order,
 * tau = u * S, token = first j whose inclusive prefix C_j exceeds tau.
 * Also returns the log-margin of the draw: the log-ratio distance of tau to
 * the two edges of the chosen bin, min(log(tau / C_{j-1}), log(C_j / tau)),
 * with C_{-1} = 0 giving +inf, and 0 when tau == 0.
 * *alt (may be NULL) receives the token on the other side of the nearer edge:
 * the last index below j with positive weight when tau is nearer C_{j-1}, the
 * first index above j with positive weight when it is nearer C_j (ties go to
 * the lower edge); -1 when there is none. A draw taken in another rounding
 * order can only move to that token when its margin is tiny.
 * Returns -1 when S <= 0.
 */
int oracle_inverse_cdf_alt(const double *r, int vocab, double u, double *margin, int32_t *alt)
{
    double total = 0.0;
    for (int v = 0; v < vocab; ++v)
        total += r[v];
    if (margin)
        *margin = 0.0;
    if (alt)
        *alt = -1;
    if (!(total > 0.0))
        return -1;
    double tau = u * total;
    double prefix = 0.0;
    for (int j = 0; j < vocab; ++j) {
        double before = prefix;
        prefix += r[j];
        if (prefix > tau) {
            double lower = INFINITY, upper = INFINITY;
            if (tau > 0.0) {
                lower = before > 0.0 ? log(tau / before) : INFINITY;
                upper = log(prefix / tau);
            } else {
                lower = before > 0.0 ? 0.0 : INFINITY;
                upper = 0.0;
            }
            if (margin)
                *margin = tau == 0.0 ? 0.0 : (lower < upper ? lower : upper);
            if (alt) {
                if (lower <= upper) {
                    for (int v = j - 1; v >= 0; --v)
                        if (r[v] > 0.0) {
                            *alt = v;
                            break;
                        }
                } else {
                    for (int v = j + 1; v < vocab; ++v)
                        if (r[v] > 0.0) {
                            *alt = v;
                            break;
                        }
                }
            }
            return j;
        }
    }
    /* unreachable: tau < total and the last prefix equals total */
    return -1;
}

int oracle_inverse_cdf(const double *r, int vocab, double u, double *margin)
{
    return oracle_inverse_cdf_alt(r, vocab, u, margin, NULL);
}

/* ----------------------------------------------------- the verification -- */

static int temperature_valid(float t, float *inv_t_out)
{
    if (isnan(t) || t < 0.0f || isinf(t))
        return 0;
    if (t == 0.0f) {
        *inv_t_out = 0.0f;
        return 1;
    }
    float inv_t = 1.0f / t;
    if (isinf(inv_t))
        return 0;
    *inv_t_out = inv_t;
    return 1;
}

/*
 * The extra token at position k of one sequence (k < gamma: the residual
 * max(0, p_k - q_k); bonus: p_k itself) from the log-normalisers of its rows,
 * by the inverse CDF of R7 at uniform u, with the fallback of R8. Element
 * offsets of the two rows are q0 (unused for the bonus) and p0.
 */
static int residual_draw(int vocab, int dtype, const void *logits_draft, size_t q0,
                         const void *logits_target, size_t p0, int bonus, float inv_t,
                         double lse_q, double lse_p, double u, double *margin, int32_t *alt)
{
    const int V = vocab;
    double *r = (double *)calloc((size_t)V, sizeof(double));
    for (int v = 0; v < V; ++v) {
        double xp = scaled(raw_logit(logits_target, dtype, p0 + (size_t)v), inv_t);
        double p = exp(xp - lse_p);
        if (!bonus) {
            double xq = scaled(raw_logit(logits_draft, dtype, q0 + (size_t)v), inv_t);
            double q = exp(xq - lse_q);
            r[v] = p - q > 0.0 ? p - q : 0.0;
        } else {
            r[v] = p;
        }
    }
    int j = oracle_inverse_cdf_alt(r, V, u, margin, alt);
    if (j < 0 && !bonus) {
        /* R8: empty residual, draw from p at the same position instead. */
        for (int v = 0; v < V; ++v) {
            double xp = scaled(raw_logit(logits_target, dtype, p0 + (size_t)v), inv_t);
            r[v] = exp(xp - lse_p);
        }
        j = oracle_inverse_cdf_alt(r, V, u, margin, alt);
    }
    free(r);
    return j;
}

/*
 * One sequence, with its uniforms given explicitly (the Philox draw is done by
 * the caller, so a test can sweep them). u_acc[i] for i < gamma and u_res[i]
 * for i <= gamma. x_q rows are draft positions 0..gamma-1, x_p rows target
 * positions 0..gamma. Element offsets of row i are q_row0 + i*V, p_row0 + i*V.
 *
 * Outputs: *accept_len, tokens[0..gamma], lse[0..2*gamma] (draft rows first,
 * then target rows; NaN where not computed), acc_margin[0..gamma-1]
 * ((lp - lq) - log u for evaluated positions, NaN elsewhere), *res_margin and
 * *res_alt (may be NULL): the token across the nearer edge of the draw's bin
 * (oracle_inverse_cdf_alt), -1 for greedy and sentinel sequences.
 */
void oracle_verify_sequence(int gamma, int vocab, int dtype,
                            const void *logits_draft, size_t q_row0,
                            const void *logits_target, size_t p_row0,
                            const int32_t *draft_tokens, float temperature,
                            const double *u_acc, const double *u_res,
                            int32_t *accept_len, int32_t *tokens,
                            double *lse, double *acc_margin, double *res_margin,
                            int32_t *res_alt)
{
    const int G = gamma, V = vocab;
    if (res_alt)
        *res_alt = -1;
    for (int i = 0; i <= G; ++i)
        tokens[i] = -1;
    for (int i = 0; i < 2 * G + 1; ++i)
        lse[i] = NAN;
    for (int i = 0; i < G; ++i)
        acc_margin[i] = NAN;
    *res_margin = NAN;
    *accept_len = -1;

    float inv_t = 0.0f;
    if (!temperature_valid(temperature, &inv_t))
        return;
    for (int i = 0; i < G; ++i)
        if (draft_tokens[i] < 0 || draft_tokens[i] >= V)
            return;

    if (temperature == 0.0f) {
        /* R4: greedy verification on raw target logits. */
        int *amax = (int *)malloc(sizeof(int) * (size_t)(G + 1));
        for (int i = 0; i <= G; ++i) {
            amax[i] = oracle_row_argmax(logits_target, dtype, p_row0 + (size_t)i * V, V);
            if (amax[i] < 0) {
                free(amax);
                return;
            }
        }
        int k = G;
        for (int i = 0; i < G; ++i) {
            if (draft_tokens[i] != amax[i]) {
                k = i;
                break;
            }
        }
        for (int i = 0; i < k; ++i)
            tokens[i] = draft_tokens[i];
        tokens[k] = amax[k];
        *accept_len = k;
        *res_margin = INFINITY;
        free(amax);
        return;
    }

    /* Log-normalisers of every row this sequence uses. */
    double *lse_q = lse;          /* [G]   */
    double *lse_p = lse + G;      /* [G+1] */
    for (int i = 0; i < G; ++i)
        lse_q[i] = oracle_row_lse(logits_draft, dtype, q_row0 + (size_t)i * V, V, inv_t);
    for (int i = 0; i <= G; ++i)
        lse_p[i] = oracle_row_lse(logits_target, dtype, p_row0 + (size_t)i * V, V, inv_t);
    for (int i = 0; i < 2 * G + 1; ++i)
        if (!(lse[i] > -INFINITY))
            return;

    /* Gather two log-probabilities per draft token, then the log-space test
     * log u < log p - log q, evaluated with IEEE semantics for -inf. */
    int k = G;
    for (int i = 0; i < G; ++i) {
        int t = draft_tokens[i];
        double xq = scaled(raw_logit(logits_draft, dtype, q_row0 + (size_t)i * V + t), inv_t);
        double xp = scaled(raw_logit(logits_target, dtype, p_row0 + (size_t)i * V + t), inv_t);
        double lq = xq - lse_q[i];
        double lp = xp - lse_p[i];
        double log_u = log(u_acc[i]);
        acc_margin[i] = (lp - lq) - log_u;
        int accept = log_u < (lp - lq);
        if (!accept) {
            k = i;
            break;
        }
    }

    /* Residual max(0, p - q) at the first rejection, or p at gamma (bonus). */
    double margin = 0.0;
    int32_t alt = -1;
    int j = residual_draw(V, dtype, logits_draft, q_row0 + (size_t)k * V, logits_target,
                          p_row0 + (size_t)k * V, k == G, inv_t, k < G ? lse_q[k] : 0.0,
                          lse_p[k], u_res[k], &margin, &alt);

    for (int i = 0; i < k; ++i)
        tokens[i] = draft_tokens[i];
    tokens[k] = j;
    *accept_len = k;
    *res_margin = margin;
    if (res_alt)
        *res_alt = alt;
}

/*
 * The batched call. seq_ids (may be NULL, meaning 0..B-1) gives the global
 * sequence index used in the Philox counter, so a sample of sequences taken
 * out of a larger batch is verified with the uniforms the full batch uses.
 * Array shapes: draft [B, G, V], target [B, G+1, V], draft_tokens [B, G],
 * temperature [B], accept_len [B], tokens [B, G+1], lse [B, 2G+1],
 * acc_margin [B, G] (may be NULL iff G == 0), res_margin [B], res_alt [B]
 * (may be NULL).
 */
void oracle_verify(int batch, int gamma, int vocab, int dtype,
                   const void *logits_draft, const void *logits_target,
                   const int32_t *draft_tokens, const float *temperature,
                   uint64_t seed, uint64_t offset, const int64_t *seq_ids,
                   int32_t *accept_len, int32_t *tokens, double *lse,
                   double *acc_margin, double *res_margin, int32_t *res_alt)
{
    const int G = gamma;
    double *u_acc = (double *)malloc(sizeof(double) * (size_t)(G + 1));
    double *u_res = (double *)malloc(sizeof(double) * (size_t)(G + 1));
    double dummy_margin[1];
    for (int b = 0; b < batch; ++b) {
        int64_t gb = seq_ids ? seq_ids[b] : (int64_t)b;
        for (int i = 0; i <= G; ++i) {
            uint32_t w[4];
            oracle_philox_words(seed, offset, gb, i, w);
            u_acc[i] = oracle_uniform24(w[0]);
            u_res[i] = oracle_uniform24(w[1]);
        }
        oracle_verify_sequence(G, vocab, dtype,
                               logits_draft, (size_t)b * G * vocab,
                               logits_target, (size_t)b * (G + 1) * vocab,
                               draft_tokens + (size_t)b * G, temperature[b],
                               u_acc, u_res, accept_len + b,
                               tokens + (size_t)b * (G + 1),
                               lse + (size_t)b * (2 * G + 1),
                               G > 0 ? acc_margin + (size_t)b * G : dummy_margin,
                               res_margin + b, res_alt ? res_alt + b : NULL);
    }
    free(u_acc);
    free(u_res);
}

/*
 * The extra token one sequence would emit if its first rejection were at
 * position k (k < gamma), or the bonus token (k == gamma), at uniform u: the
 * residual draw of the verification (R7, R8) on the rows of position k alone.
 * Rows: draft row at element offset q0 (unused when k == gamma), target row
 * at p0. temperature must be > 0. Outputs the token (or -1 when a row has no
 * finite logit), its log-margin and the token across the nearer bin edge.
 */
void oracle_draw_at(int vocab, int dtype, const void *logits_draft, size_t q0,
                    const void *logits_target, size_t p0, int bonus, float temperature,
                    double u, int32_t *token, double *margin, int32_t *alt)
{
    float inv_t = 0.0f;
    *token = -1;
    *margin = NAN;
    *alt = -1;
    if (!temperature_valid(temperature, &inv_t) || !(temperature > 0.0f))
        return;
    double lse_p = oracle_row_lse(logits_target, dtype, p0, vocab, inv_t);
    double lse_q = bonus ? 0.0 : oracle_row_lse(logits_draft, dtype, q0, vocab, inv_t);
    if (!(lse_p > -INFINITY) || !(lse_q > -INFINITY))
        return;
    *token = residual_draw(vocab, dtype, logits_draft, q0, logits_target, p0, bonus, inv_t,
                           lse_q, lse_p, u, margin, alt);
}

/*
 * Scalar-only mode: the gathered pairs logprobs[b, i, 0] = log q (draft) and
 * logprobs[b, i, 1] = log p (target), temperature already applied upstream
 * (FlashSpec summary, Methodology section 1: two log-probability scalars per
 * candidate, one from each model; traffic O(B*gamma)). Same counters and the
 * same accept test as the full call; only the accept length is produced.
 */
void oracle_accept_logprobs(int batch, int gamma, const float *logprobs,
                            uint64_t seed, uint64_t offset, const int64_t *seq_ids,
                            int32_t *accept_len, double *acc_margin)
{
    const int G = gamma;
    for (int b = 0; b < batch; ++b) {
        int64_t gb = seq_ids ? seq_ids[b] : (int64_t)b;
        int k = G;
        for (int i = 0; i < G; ++i)
            acc_margin[(size_t)b * G + i] = NAN;
        for (int i = 0; i < G; ++i) {
            uint32_t w[4];
            oracle_philox_words(seed, offset, gb, i, w);
            double log_u = log(oracle_uniform24(w[0]));
            double lq = (double)logprobs[((size_t)b * G + i) * 2 + 0];
            double lp = (double)logprobs[((size_t)b * G + i) * 2 + 1];
            acc_margin[(size_t)b * G + i] = (lp - lq) - log_u;
            if (!(log_u < (lp - lq))) {
                k = i;
                break;
            }
        }
        accept_len[b] = k;
    }
}

/*
 * The gathered pairs themselves, as the full call sees them: for every
 * sequence with T > 0 that is valid, out[b, i, 0] = x_q[i][t_i] - lse_q[i] and
 * out[b, i, 1] = x_p[i][t_i] - lse_p[i] in double; NaN for other sequences.
 */
void oracle_gather_logprobs(int batch, int gamma, int vocab, int dtype,
                            const void *logits_draft, const void *logits_target,
                            const int32_t *draft_tokens, const float *temperature,
                            double *out)
{
    const int G = gamma, V = vocab;
    for (int b = 0; b < batch; ++b) {
        float inv_t = 0.0f;
        int ok = temperature_valid(temperature[b], &inv_t) && temperature[b] > 0.0f;
        for (int i = 0; i < G && ok; ++i)
            if (draft_tokens[(size_t)b * G + i] < 0 || draft_tokens[(size_t)b * G + i] >= V)
                ok = 0;
        for (int i = 0; i < G; ++i) {
            double *o = out + ((size_t)b * G + i) * 2;
            o[0] = o[1] = NAN;
            if (!ok)
                continue;
            int t = draft_tokens[(size_t)b * G + i];
            size_t q0 = ((size_t)b * G + i) * V, p0 = ((size_t)b * (G + 1) + i) * V;
            double lq = oracle_row_lse(logits_draft, dtype, q0, V, inv_t);
            double lp = oracle_row_lse(logits_target, dtype, p0, V, inv_t);
            o[0] = (double)scaled(raw_logit(logits_draft, dtype, q0 + t), inv_t) - lq;
            o[1] = (double)scaled(raw_logit(logits_target, dtype, p0 + t), inv_t) - lp;
        }
    }
}

/* ----------------------------------------------- verification outcomes -- */

/*
 * The distribution of one verification's outcome, given the drafted tokens.
 * The outcome of a verification is the pair (accepted count k, extra token)
 * that speculative speculative decoding predicts and keys its speculation
 * cache on; its Saguaro algorithm spends the cache on the most likely lengths
 * and, per length, on the F most likely extra tokens of the residual
 * distribution (Speculative Speculative Decoding summary, section 2: central
 * concept items 1-3; Saguaro challenge 1, fan-out over likely lengths;
 * challenge 2, the top-F tokens of the residual the bonus token is drawn from).
 * Under the rule of this file, with the drafts t fixed:
 *   beta_j = min(1, p_j(t_j) / q_j(t_j)), evaluated as min(1, exp(lp_j - lq_j))
 *            (0 when lp_j - lq_j is NaN, the reject case of the test);
 *   P(k = i | t) = prod_{j<i} beta_j * (1 - beta_i) for i < gamma,
 *   P(k = gamma | t) = prod_{j<gamma} beta_j;
 *   extra token | k = i  ~  r_i / S_i, r_i = max(0, p_i - q_i) for i < gamma,
 *                           r_gamma = p_gamma; r_i = p_i when S_i == 0 (R8).
 * Readings: R21 the list for length i holds the F tokens of largest r_i(v),
 *   ties to the lowest index, padded with token -1 / probability 0 when V < F;
 *   R22 greedy sequences (T == 0) have a deterministic outcome: the list holds
 *   the F largest raw target logits (argmax first) with probabilities 1, 0, ...
 *   and P(k = i | t) is 0 or 1;
 *   R23 out_mass[i] = S_i = sum_v max(0, p_i - q_i), the total-variation
 *   distance of p_i and q_i (so 1 - S_i is the acceptance probability of
 *   position i averaged over the draft token); 1 at i = gamma; 0 for greedy;
 *   sentinel sequences (as in the verification) get tokens -1 and zeros.
 *
 * Shapes: out_tok / out_prob [B][G+1][F], out_pk / out_mass [B][G+1];
 * out_dist and out_scale [B][G+1][V] may be NULL: when given they receive the
 * whole distribution r_i / S_i and the magnitude (p_i + q_i) / S_i of the two
 * terms behind each entry (p_i / S_i at i = gamma, 0 for greedy).
 */
void oracle_outcomes(int batch, int gamma, int vocab, int dtype,
                     const void *logits_draft, const void *logits_target,
                     const int32_t *draft_tokens, const float *temperature, int F,
                     int32_t *out_tok, double *out_prob, double *out_pk, double *out_mass,
                     double *out_dist, double *out_scale)
{
    const int G = gamma, V = vocab;
    double *r = (double *)malloc(sizeof(double) * (size_t)V);
    double *sc = (double *)malloc(sizeof(double) * (size_t)V);
    double *lse_q = (double *)malloc(sizeof(double) * (size_t)(G + 1));
    double *lse_p = (double *)malloc(sizeof(double) * (size_t)(G + 1));
    double *beta = (double *)malloc(sizeof(double) * (size_t)(G + 1));
    char *taken = (char *)malloc((size_t)V);
    for (int b = 0; b < batch; ++b) {
        const size_t q_row0 = (size_t)b * G * V, p_row0 = (size_t)b * (G + 1) * V;
        const int32_t *t = draft_tokens + (size_t)b * G;
        int32_t *tok_b = out_tok + (size_t)b * (G + 1) * F;
        double *prob_b = out_prob + (size_t)b * (G + 1) * F;
        double *pk_b = out_pk + (size_t)b * (G + 1);
        double *mass_b = out_mass + (size_t)b * (G + 1);
        for (int i = 0; i < (G + 1) * F; ++i) {
            tok_b[i] = -1;
            prob_b[i] = 0.0;
        }
        for (int i = 0; i <= G; ++i) {
            pk_b[i] = 0.0;
            mass_b[i] = 0.0;
        }
        if (out_dist)
            memset(out_dist + (size_t)b * (G + 1) * V, 0, sizeof(double) * (size_t)(G + 1) * V);
        if (out_scale)
            memset(out_scale + (size_t)b * (G + 1) * V, 0, sizeof(double) * (size_t)(G + 1) * V);

        /* validity, as in the verification (sentinel rule) */
        float inv_t = 0.0f;
        int ok = temperature_valid(temperature[b], &inv_t);
        for (int i = 0; ok && i < G; ++i)
            if (t[i] < 0 || t[i] >= V)
                ok = 0;
        const int greedy = ok && temperature[b] == 0.0f;
        if (ok && greedy) {
            for (int i = 0; i <= G && ok; ++i)
                if (oracle_row_argmax(logits_target, dtype, p_row0 + (size_t)i * V, V) < 0)
                    ok = 0;
        } else if (ok) {
            for (int i = 0; i < G; ++i)
                lse_q[i] = oracle_row_lse(logits_draft, dtype, q_row0 + (size_t)i * V, V, inv_t);
            for (int i = 0; i <= G; ++i)
                lse_p[i] = oracle_row_lse(logits_target, dtype, p_row0 + (size_t)i * V, V, inv_t);
            for (int i = 0; i < G; ++i)
                if (!(lse_q[i] > -INFINITY))
                    ok = 0;
            for (int i = 0; i <= G; ++i)
                if (!(lse_p[i] > -INFINITY))
                    ok = 0;
        }
        if (!ok)
            continue;

        /* per-position acceptance probability of the drafted token */
        for (int j = 0; j < G; ++j) {
            if (greedy) {
                beta[j] = t[j] == oracle_row_argmax(logits_target, dtype,
                                                    p_row0 + (size_t)j * V, V) ? 1.0 : 0.0;
            } else {
                double xq = scaled(raw_logit(logits_draft, dtype, q_row0 + (size_t)j * V + t[j]), inv_t);
                double xp = scaled(raw_logit(logits_target, dtype, p_row0 + (size_t)j * V + t[j]), inv_t);
                double d = (xp - lse_p[j]) - (xq - lse_q[j]);
                beta[j] = d >= 0.0 ? 1.0 : (d < 0.0 ? exp(d) : 0.0);
            }
        }
        double reach = 1.0; /* P(k >= i | t) */
        for (int i = 0; i <= G; ++i) {
            pk_b[i] = i < G ? reach * (1.0 - beta[i]) : reach;
            if (i < G)
                reach *= beta[i];
        }

        for (int i = 0; i <= G; ++i) {
            /* the distribution of the extra token at length i */
            double S = 0.0;
            if (greedy) {
                for (int v = 0; v < V; ++v) {
                    r[v] = raw_logit(logits_target, dtype, p_row0 + (size_t)i * V + v);
                    sc[v] = 0.0;
                }
            } else {
                for (int v = 0; v < V; ++v) {
                    double xp = scaled(raw_logit(logits_target, dtype, p_row0 + (size_t)i * V + v), inv_t);
                    double p = exp(xp - lse_p[i]);
                    if (i < G) {
                        double xq = scaled(raw_logit(logits_draft, dtype, q_row0 + (size_t)i * V + v), inv_t);
                        double q = exp(xq - lse_q[i]);
                        r[v] = p - q > 0.0 ? p - q : 0.0;
                        sc[v] = p + q;
                    } else {
                        r[v] = p;
                        sc[v] = p;
                    }
                    S += r[v];
                }
                mass_b[i] = i < G ? S : 1.0;
                if (!(S > 0.0)) {
                    /* R8: an empty residual means the draw comes from p_i */
                    S = 0.0;
                    for (int v = 0; v < V; ++v) {
                        double xp = scaled(raw_logit(logits_target, dtype, p_row0 + (size_t)i * V + v), inv_t);
                        r[v] = exp(xp - lse_p[i]);
                        sc[v] = r[v];
                        S += r[v];
                    }
                }
            }
            /* the F largest entries, lowest index first among equals */
            memset(taken, 0, (size_t)V);
            int n = F < V ? F : V;
            for (int j = 0; j < n; ++j) {
                int best = -1;
                for (int v = 0; v < V; ++v) {
                    if (taken[v])
                        continue;
                    if (best < 0 || r[v] > r[best])
                        best = v;
                }
                taken[best] = 1;
                tok_b[(size_t)i * F + j] = best;
                prob_b[(size_t)i * F + j] = greedy ? (j == 0 ? 1.0 : 0.0) : r[best] / S;
            }
            if (out_dist) {
                double *dd = out_dist + ((size_t)b * (G + 1) + i) * V;
                double *ss = out_scale ? out_scale + ((size_t)b * (G + 1) + i) * V : NULL;
                if (greedy) {
                    dd[tok_b[(size_t)i * F]] = 1.0;
                } else {
                    for (int v = 0; v < V; ++v) {
                        dd[v] = r[v] / S;
                        if (ss)
                            ss[v] = sc[v] / S;
                    }
                }
            }
        }
    }
    free(r);
    free(sc);
    free(lse_q);
    free(lse_p);
    free(beta);
    free(taken);
}

/*
 * Speculation-cache budget per length (Speculative Speculative Decoding
 * summary, section 2, Saguaro challenge 1: the cache budget is spread over
 * the lengths unevenly, more speculations for likely lengths and fewer for
 * unlikely ones, so that a fixed budget hits the cache as often as it can;
 * the page names a geometric allocation and gives no formula).
 * Reading R25: a cache entry is a pair (length i, the j-th token of length
 * i's list), worth v(i, j) = P(k = i) * P(extra = token_j | k = i), the
 * probability that the verification outcome is that pair; v is taken as 0
 * when the product is negative or NaN. The budget is handed out one entry at
 * a time, each to the length whose next unused list entry is worth the most,
 * the lower length on equal worth, until `budget` entries are placed or every
 * list is used up. Each length thus gets a prefix of its list, n_i entries;
 * when every list is non-increasing (as spec_verify_outcomes writes them) the
 * placed entries are the `budget` most valuable pairs, which maximises the
 * expected hit rate sum v over the cache. The page's geometric allocation is
 * the case P(k = i) proportional to alpha^i of a fixed acceptance rate alpha.
 * out_hit is the sum of the placed values in the order they were placed.
 * Products and sums in double (a product of two floats is exact in double).
 * Shapes: pk [B][L], probs [B][L][F], out_n [B][L], out_hit [B] (may be NULL).
 */
void oracle_outcome_fanout(int batch, int lengths, int F, const float *pk, const float *probs,
                           int budget, int32_t *out_n, double *out_hit)
{
    const int L = lengths;
    for (int b = 0; b < batch; ++b) {
        const float *pk_b = pk + (size_t)b * L;
        const float *pr_b = probs + (size_t)b * L * F;
        int32_t *n = out_n + (size_t)b * L;
        for (int i = 0; i < L; ++i)
            n[i] = 0;
        double hit = 0.0;
        for (int step = 0; step < budget; ++step) {
            int best = -1;
            double best_v = 0.0;
            for (int i = 0; i < L; ++i) {
                if (n[i] >= F)
                    continue;
                double v = (double)pk_b[i] * (double)pr_b[(size_t)i * F + n[i]];
                if (!(v > 0.0))
                    v = 0.0;
                if (best < 0 || v > best_v) {
                    best = i;
                    best_v = v;
                }
            }
            if (best < 0)
                break; /* every list is used up */
            n[best] += 1;
            hit += best_v;
        }
        if (out_hit)
            out_hit[b] = hit;
    }
}

/* ------------------------------------------------ low-rank draft head -- */

/* binary32 -> bfloat16, round to nearest even (finite inputs). */
static uint16_t oracle_bf16_rne(double x)
{
    float f = (float)x; /* a first guess only: bf16_nearest checks it */
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* The bfloat16 nearest to x (ties to even), decided in double: the two
 * neighbours of x on the bfloat16 grid are compared by their distance. */
static uint16_t bf16_nearest(double x)
{
    uint16_t c = oracle_bf16_rne(x); /* a candidate within one step */
    double best = (double)bf16_bits_to_float(c);
    uint16_t out = c;
    for (int d = -1; d <= 1; d += 2) {
        uint16_t n = (uint16_t)(c + d);
        double v = (double)bf16_bits_to_float(n);
        double e0 = fabs(best - x), e1 = fabs(v - x);
        if (e1 < e0 || (e1 == e0 && (n & 1u) == 0u)) {
            best = v;
            out = n;
        }
    }
    return out;
}

/*
 * The low-rank draft LM head and the normaliser of its logits. The SlimSpec
 * summary (Methodology, architecture) replaces the draft's full projection
 * z = W_full h by z = W_up W_down h with W_down in R^{r x d}, W_up in
 * R^{V x r}, r << d, computed with dense matrix products. Readings:
 *   SL1 h, W_down and W_up are bfloat16; the rank-r activation u = W_down h is
 *       a bfloat16 tensor (the output of a bf16 linear layer, rounded to
 *       nearest even), and the logits z = W_up u are rounded to bfloat16 (the
 *       dtype the verifier reads);
 *   SL2 the normaliser is that of the verifier's draft rows (R3):
 *       lse = log sum_v exp(fl32(z_v * fl32(1/T))), NaN when T is not > 0 or
 *       the reciprocal overflows.
 * Products and sums are exact up to the rounding of double (each product of
 * two bfloat16 values is exact; sums of at most 2^16 terms of such products
 * carry a relative error below 2^-37 of their magnitude), so the roundings to
 * bfloat16 are those of the exact values except within that margin.
 *
 * Outputs (row-major): u_exact [N][r], u [N][r] (bf16 bits), u_abs [N][r]
 * = sum_k |W_down[j][k] h[k]|; z_exact [N][V] = W_up u (from the rounded u),
 * z [N][V] (bf16 bits), z_abs [N][V] = sum_j |W_up[v][j] u[j]|; lse [N].
 * rows restricts the work to a subset of rows (NULL = all): row i of the
 * outputs is input row rows[i].
 */
void oracle_lowrank_head(int n_rows, int d, int r, int V, const uint16_t *h,
                         const uint16_t *w_down, const uint16_t *w_up, const float *temperature,
                         const int32_t *rows, double *u_exact, uint16_t *u, double *u_abs,
                         double *z_exact, uint16_t *z, double *z_abs, double *lse)
{
    double *uu = (double *)malloc(sizeof(double) * (size_t)r);
    for (int i = 0; i < n_rows; ++i) {
        const int row = rows ? rows[i] : i;
        const uint16_t *hr = h + (size_t)row * d;
        for (int j = 0; j < r; ++j) {
            double s = 0.0, a = 0.0;
            for (int k = 0; k < d; ++k) {
                double t = (double)bf16_bits_to_float(w_down[(size_t)j * d + k]) *
                           (double)bf16_bits_to_float(hr[k]);
                s += t;
                a += fabs(t);
            }
            u_exact[(size_t)i * r + j] = s;
            u_abs[(size_t)i * r + j] = a;
            u[(size_t)i * r + j] = bf16_nearest(s);
            uu[j] = (double)bf16_bits_to_float(u[(size_t)i * r + j]);
        }
        for (int v = 0; v < V; ++v) {
            double s = 0.0, a = 0.0;
            for (int j = 0; j < r; ++j) {
                double t = (double)bf16_bits_to_float(w_up[(size_t)v * r + j]) * uu[j];
                s += t;
                a += fabs(t);
            }
            z_exact[(size_t)i * V + v] = s;
            z_abs[(size_t)i * V + v] = a;
            z[(size_t)i * V + v] = bf16_nearest(s);
        }
        float inv_t = 0.0f;
        if (!temperature_valid(temperature[row], &inv_t) || temperature[row] == 0.0f) {
            lse[i] = NAN;
            continue;
        }
        lse[i] = oracle_row_lse(z + (size_t)i * V, ORACLE_BF16, 0, V, inv_t);
    }
    free(uu);
}

/* ------------------------------------------------------------ draft trees -- */

/*
 * Confidence-guided pruning of a batch of draft trees (SpecLA summary,
 * Methodology section 3, target-aligned drafting: low-probability paths are
 * pruned by their cumulative log-probability before verification).
 * Tree b has M nodes in topological order: node 0 is the root (the last
 * verified token, no draft token), and node i >= 1 hangs under parent[i] in
 * [0, i) with its draft token's log-probability logq[i] <= 0 given its path.
 * Readings:
 *   TR1 the path score is c(0) = 0, c(i) = c(parent(i)) + logq(i), added from
 *       the root down in double;
 *   TR2 a node is kept iff c(i) >= tau and it is among the K nodes with the
 *       largest c (ties to the lower index). Both sets are closed under
 *       ancestors because scores never rise along a path, so every kept node's
 *       path is kept; the root is always kept (K >= 1, tau <= 0);
 *   TR3 a tree whose parent array is not topological, or with a log-probability
 *       that is NaN or positive, is a sentinel: count -1, nothing kept.
 * Outputs: cum [B][M] (NaN for sentinel trees), new_index [B][M] (position of
 * the node among the kept ones in index order, -1 if pruned), new_parent
 * [B][M] (by new position: the parent's new index, -1 for the root and for
 * unused slots), count [B].
 */
void oracle_tree_prune(int B, int M, const int32_t *parent, const float *logq, double tau,
                       int K, double *cum, int32_t *new_index, int32_t *new_parent,
                       int32_t *count)
{
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parent + (size_t)b * M;
        const float *lq = logq + (size_t)b * M;
        double *c = cum + (size_t)b * M;
        int32_t *ni = new_index + (size_t)b * M;
        int32_t *np = new_parent + (size_t)b * M;
        int ok = par[0] == -1;
        for (int i = 1; i < M && ok; ++i)
            if (par[i] < 0 || par[i] >= i || isnan(lq[i]) || lq[i] > 0.0f)
                ok = 0;
        for (int i = 0; i < M; ++i) {
            ni[i] = -1;
            np[i] = -1;
            c[i] = NAN;
        }
        if (!ok) {
            count[b] = -1;
            continue;
        }
        c[0] = 0.0;
        for (int i = 1; i < M; ++i)
            c[i] = c[par[i]] + (double)lq[i];
        int n = 0;
        for (int i = 0; i < M; ++i) {
            /* rank of node i: how many nodes score higher (ties: lower index) */
            int rank = 0;
            for (int j = 0; j < M; ++j)
                if (c[j] > c[i] || (c[j] == c[i] && j < i))
                    ++rank;
            if (c[i] >= tau && rank < K)
                ni[i] = n++;
        }
        for (int i = 0; i < M; ++i)
            if (ni[i] >= 0)
                np[ni[i]] = i == 0 ? -1 : ni[par[i]];
        count[b] = n;
    }
}

/*
 * Greedy verification of a batch of (pruned) draft trees: at T = 0 a draft
 * token is accepted when it equals the target's argmax after its parent, and a
 * tree is accepted along the path that keeps matching (the exact-match rule of
 * token-tree speculative decoding, e.g. Miao et al., SpecInfer, ASPLOS 2024;
 * on a chain it is the greedy rule R4 of the verifier). Readings:
 *   TR4 the target's logits are given for every node, row i holding the
 *       distribution of the token that follows node i's path; a[i] is its
 *       argmax over raw logits, lowest index on ties;
 *   TR5 from the root, step to the lowest-index child whose token is a[x] while
 *       there is one; the extra token is a[last node];
 *   TR6 trees with n nodes < 1 or > M, a parent outside [0, i), a token
 *       outside [0, V), or a row of a reached node with no finite logit get
 *       length -1, path -1, extra token -1.
 * Shapes: parent, token [B][M] (node 0's token is ignored), n_nodes [B],
 * target [B][M][V]; outputs length [B], path [B][M] (accepted nodes in order,
 * -1 padded), extra [B].
 */
void oracle_tree_verify_greedy(int B, int M, int V, int dtype, const int32_t *parent,
                               const int32_t *token, const int32_t *n_nodes, const void *target,
                               int32_t *length, int32_t *path, int32_t *extra)
{
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parent + (size_t)b * M;
        const int32_t *tk = token + (size_t)b * M;
        int32_t *pa = path + (size_t)b * M;
        const int n = n_nodes[b];
        for (int i = 0; i < M; ++i)
            pa[i] = -1;
        length[b] = -1;
        extra[b] = -1;
        int ok = n >= 1 && n <= M && par[0] == -1;
        for (int i = 1; i < n && ok; ++i)
            if (par[i] < 0 || par[i] >= i || tk[i] < 0 || tk[i] >= V)
                ok = 0;
        if (!ok)
            continue;
        int x = 0, L = 0;
        for (;;) {
            int a = oracle_row_argmax(target, dtype, ((size_t)b * M + x) * V, V);
            if (a < 0) {
                L = -1;
                break;
            }
            int next = -1;
            for (int j = 1; j < n; ++j)
                if (par[j] == x && tk[j] == a) {
                    next = j;
                    break;
                }
            if (next < 0) {
                extra[b] = a;
                break;
            }
            pa[L++] = next;
            x = next;
        }
        if (L < 0) {
            for (int i = 0; i < M; ++i)
                pa[i] = -1;
            continue;
        }
        length[b] = L;
    }
}

/*
 * Sampled verification of a batch of draft trees (T > 0): multi-step
 * speculative sampling (Miao et al., SpecInfer, ASPLOS 2024, its tree
 * verification with stochastic decoding), written here with one draft
 * distribution per node: the children of node u are draft tokens drawn
 * independently from q_u. The pages name tree drafting and pruning but give no
 * multi-branch acceptance rule; this is the published one that keeps the
 * target's output distribution. Readings:
 *   TS1 rows: target row u holds the distribution of the token that follows
 *       node u's path (p_u), draft row u the distribution u's children were
 *       drawn from (q_u); x = fl32(z * fl32(1/T)) as in R3;
 *   TS2 at node u with current target pi (pi = p_u on arrival), u's children
 *       are tried in increasing node order; child s with token t is accepted
 *       iff log u_acc(s) < log pi(t) - log q_u(t) (IEEE, as in R5); on
 *       acceptance the walk moves to s with pi = p_s; on rejection
 *       pi <- max(0, pi - q_u) / its sum, unless that sum is <= 0 (rounding
 *       only), when pi stays (as in R8);
 *   TS3 when u has no child left to try (all rejected, or none) the extra token
 *       is drawn from pi by the inverse CDF of R7;
 *   TS4 uniforms: Philox block (s - 1, b) word 0 is child s's accept uniform,
 *       block (L, b) word 1 the draw's, L the number of accepted nodes; on a
 *       chain (node i + 1 holding draft token i) these are the verifier's R6
 *       uniforms, and the rule is the verifier's, so a chain gives the same
 *       outcome as oracle_verify;
 *   TS5 T == 0: the greedy rule TR5 (no uniforms);
 *   TS6 sentinels: TR6's, a temperature R3 rejects, or a row the walk needs
 *       with no finite logit: length -1, path -1, extra -1.
 * Before any rejection at u, log pi(t) is x_p(t) - lse_p(u) and the residual
 * weights are max(0, p - q) unnormalised, so on a chain every operation is
 * oracle_verify_sequence's.
 * Shapes: parent, token [B][M], n_nodes [B], draft and target [B][M][V],
 * temperature [B], seq_ids [B] (NULL: 0..B-1, the b of the Philox counter);
 * outputs length [B], path [B][M], extra [B], acc_margin [B] (smallest
 * |(log pi - log q) - log u| over the tests made, +inf if none) and
 * res_margin [B] (the draw's log-margin of R7), each may be NULL.
 */
static int load_row_prob(const void *base, int dtype, size_t row0, int V, float inv_t,
                         double *lse_out, double *prob)
{
    double lse = oracle_row_lse(base, dtype, row0, V, inv_t);
    *lse_out = lse;
    if (!(lse > -INFINITY))
        return 0;
    for (int v = 0; v < V; ++v)
        prob[v] = exp((double)scaled(raw_logit(base, dtype, row0 + (size_t)v), inv_t) - lse);
    return 1;
}

void oracle_tree_verify_sample(int B, int M, int V, int dtype, const int32_t *parent,
                               const int32_t *token, const int32_t *n_nodes, const void *draft,
                               const void *target, const float *temperature, uint64_t seed,
                               uint64_t offset, const int64_t *seq_ids, int32_t *length,
                               int32_t *path, int32_t *extra, double *acc_margin,
                               double *res_margin)
{
    double *pi = (double *)malloc(sizeof(double) * (size_t)V);
    double *q = (double *)malloc(sizeof(double) * (size_t)V);
    double *w = (double *)malloc(sizeof(double) * (size_t)V);
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parent + (size_t)b * M;
        const int32_t *tk = token + (size_t)b * M;
        int32_t *pa = path + (size_t)b * M;
        const int n = n_nodes[b];
        for (int i = 0; i < M; ++i)
            pa[i] = -1;
        length[b] = -1;
        extra[b] = -1;
        if (acc_margin)
            acc_margin[b] = NAN;
        if (res_margin)
            res_margin[b] = NAN;
        int ok = n >= 1 && n <= M && par[0] == -1;
        for (int i = 1; i < n && ok; ++i)
            if (par[i] < 0 || par[i] >= i || tk[i] < 0 || tk[i] >= V)
                ok = 0;
        float inv_t = 0.0f;
        if (!ok || !temperature_valid(temperature[b], &inv_t))
            continue;
        if (temperature[b] == 0.0f) {
            /* TS5 */
            oracle_tree_verify_greedy(1, M, V, dtype, par, tk, &n_nodes[b],
                                      (const char *)target + (size_t)b * M * V * (dtype == ORACLE_BF16 ? 2 : 4),
                                      &length[b], pa, &extra[b]);
            if (length[b] >= 0) {
                if (acc_margin)
                    acc_margin[b] = INFINITY;
                if (res_margin)
                    res_margin[b] = INFINITY;
            }
            continue;
        }
        const int64_t sid = seq_ids ? seq_ids[b] : b;
        const size_t base = (size_t)b * M * V;
        int u = 0, L = 0, bad = 0;
        double amin = INFINITY;
        double lse_p = 0.0, lse_q = 0.0;
        if (!load_row_prob(target, dtype, base, V, inv_t, &lse_p, pi))
            bad = 1;
        /* weights of the current target: pi itself until a rejection, then
         * the unnormalised residual w with sum wsum */
        int residual = 0;
        double wsum = 1.0;
        while (!bad) {
            int moved = 0, have_q = 0;
            for (int s = 1; s < n && !bad; ++s) {
                if (par[s] != u)
                    continue;
                if (!have_q) {
                    if (!load_row_prob(draft, dtype, base + (size_t)u * V, V, inv_t, &lse_q, q)) {
                        bad = 1;
                        break;
                    }
                    have_q = 1;
                }
                const int t = tk[s];
                uint32_t words[4];
                oracle_philox_words(seed, offset, sid, s - 1, words);
                const double log_u = log(oracle_uniform24(words[0]));
                const double xq = scaled(raw_logit(draft, dtype, base + (size_t)u * V + t), inv_t);
                const double lq = xq - lse_q;
                double lpi;
                if (!residual) {
                    const double xp =
                        scaled(raw_logit(target, dtype, base + (size_t)u * V + t), inv_t);
                    lpi = xp - lse_p;
                } else {
                    lpi = log(w[t]) - log(wsum);
                }
                const double m = (lpi - lq) - log_u;
                if (fabs(m) < amin)
                    amin = fabs(m);
                if (log_u < lpi - lq) {
                    pa[L++] = s;
                    u = s;
                    moved = 1;
                    residual = 0;
                    wsum = 1.0;
                    if (!load_row_prob(target, dtype, base + (size_t)u * V, V, inv_t, &lse_p, pi))
                        bad = 1;
                    break;
                }
                /* rejection: pi <- max(0, pi - q_u) / sum, pi being p_u or
                 * w / wsum; the first pass only sums, so an empty residual
                 * leaves pi as it was */
                double sum = 0.0;
                for (int v = 0; v < V; ++v) {
                    const double cur = residual ? w[v] / wsum : pi[v];
                    const double r = cur - q[v];
                    sum += r > 0.0 ? r : 0.0;
                }
                if (sum > 0.0) {
                    for (int v = 0; v < V; ++v) {
                        const double cur = residual ? w[v] / wsum : pi[v];
                        const double r = cur - q[v];
                        w[v] = r > 0.0 ? r : 0.0;
                    }
                    wsum = sum;
                    residual = 1;
                }
            }
            if (!moved)
                break;
        }
        if (bad) {
            for (int i = 0; i < M; ++i)
                pa[i] = -1;
            continue;
        }
        uint32_t words[4];
        oracle_philox_words(seed, offset, sid, L, words);
        double margin = 0.0;
        const int j = oracle_inverse_cdf(residual ? w : pi, V, oracle_uniform24(words[1]), &margin);
        length[b] = L;
        extra[b] = j;
        if (acc_margin)
            acc_margin[b] = amin;
        if (res_margin)
            res_margin[b] = margin;
    }
    free(pi);
    free(q);
    free(w);
}
