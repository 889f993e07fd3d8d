/*
 * bandit_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain CPU reference for online draft-model selection: a K-armed bandit
 * whose reward is the fraction of draft tokens the verifier accepted
 * (FlashSpec technical summary, Methodology section 2, "draft selection via
 * online bandit": one arm per draft model, UCB1 or Thompson sampling, reward
 * alpha = accepted fraction; Significance section, Theorem 1: the output
 * distribution is unchanged because the policy looks only at past accept
 * counts). Same rules as spec_oracle.c: only the test suite may load it, it
 * shares nothing with the HIP library, and all arithmetic is IEEE double with
 * contraction off, in the obvious order.
 *
 * The pages name the two policies but print no formulas; the textbook forms are
 * used, each from its publication:
 *   UCB1 (Auer, Cesa-Bianchi and Fischer, Machine Learning 47, 2002, Fig. 1):
 *     play every arm once, then the arm maximising  mean_j + sqrt(2 ln n / n_j),
 *     n the number of plays so far;
 *   Thompson sampling with a Beta(1, 1) prior (Agrawal and Goyal, COLT 2012):
 *     draw theta_j ~ Beta(1 + S_j, 1 + F_j) and play the largest;
 *   Gamma variates by Marsaglia and Tsang (ACM TOMS 26(3), 2000), normal
 *     variates by Box and Muller (Ann. Math. Stat. 29, 1958), and
 *     Beta(a, b) = X / (X + Y) with X ~ Gamma(a), Y ~ Gamma(b).
 *
 * Readings taken where the pages are silent:
 *   B1 sequences are split into G groups of B/G consecutive sequences, one
 *      bandit per group (G = 1: one arm per decoding step for the whole batch;
 *      G = B: one bandit per sequence slot). One call is one round per group;
 *   B2 a group's reward is sum_b k_b / (gamma * m) over its m sequences with
 *      a valid accept length k_b in [0, gamma]; a group with m = 0 is not
 *      updated (the round does not count);
 *   B3 Thompson sampling takes the fractional reward directly: S_j = sum of
 *      rewards, F_j = n_j - S_j (with 0/1 rewards this is Beta-Bernoulli);
 *   B4 ties go to the lowest arm index; UCB1's opening plays go in index order;
 *   B5 Philox4x32-10 with key (lo32(seed), hi32(seed)) and counter
 *      (2^31 | (64 * (2 j + s) + attempt), g, lo32(offset), hi32(offset)) for
 *      arm j, s = 0 for X and 1 for Y, attempt < 64. Bit 31 keeps these
 *      counters apart from the verifier's, whose first word is a position;
 *      u1 = (w0 + 1) 2^-32, u2 = w1 2^-32, U = (w2 + 1) 2^-32;
 *   B6 Marsaglia-Tsang without the squeeze step; after 64 failed attempts
 *      (probability below 1e-80 for shape >= 1) the variate is d;
 *   B7 an arm index outside [0, K) in the played-arm input means the group is
 *      neither updated nor given an arm: its output is -1.
 *
 * Every floating-point decision reports a margin, so that a caller comparing
 * against another implementation of the same arithmetic can tell a real
 * disagreement from an ulp-level tie: UCB1 and Thompson report the relative gap
 * between the best and second-best score; Thompson also folds in the gap of
 * every accept test and every sign test inside Marsaglia-Tsang.
 */
#include <float.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#if !defined(FLT_EVAL_METHOD) || FLT_EVAL_METHOD != 0
#error "the oracle needs FLT_EVAL_METHOD == 0"
#endif

#define BANDIT_UCB1 0
#define BANDIT_THOMPSON 1
#define BANDIT_MAX_ARMS 64
#define BANDIT_MAX_ATTEMPTS 64

/* defined in spec_oracle.c (same library) */
void oracle_philox4x32_10(const uint32_t counter[4], const uint32_t key[2], uint32_t out[4]);

static double min2(double a, double b) { return a < b ? a : b; }

/* The Philox block of one Marsaglia-Tsang attempt (B5). */
static void bandit_words(uint64_t seed, uint64_t offset, int group, int arm, int which,
                         int attempt, uint32_t out[4])
{
    uint32_t key[2] = { (uint32_t)seed, (uint32_t)(seed >> 32) };
    uint32_t ctr[4] = { 0x80000000u | (uint32_t)(BANDIT_MAX_ATTEMPTS * (2 * arm + which) + attempt),
                        (uint32_t)group, (uint32_t)offset, (uint32_t)(offset >> 32) };
    oracle_philox4x32_10(ctr, key, out);
}

/*
 * Gamma(shape, 1) for shape >= 1 by Marsaglia and Tsang: with d = shape - 1/3
 * and c = 1/sqrt(9 d), draw a standard normal z and a uniform U; with
 * v = (1 + c z)^3, accept d v when v > 0 and ln U < z^2/2 + d - d v + d ln v.
 * The normal is Box-Muller's cosine branch. *margin is lowered to the smallest
 * relative gap of any test taken.
 */
double oracle_gamma_mt(double shape, uint64_t seed, uint64_t offset, int group, int arm,
                       int which, double *margin)
{
    const double d = shape - 1.0 / 3.0;
    const double c = 1.0 / sqrt(9.0 * d);
    const double two_pi = 6.283185307179586;
    const double scale = d > 1.0 ? d : 1.0;
    for (int attempt = 0; attempt < BANDIT_MAX_ATTEMPTS; ++attempt) {
        uint32_t w[4];
        bandit_words(seed, offset, group, arm, which, attempt, w);
        double u1 = ((double)w[0] + 1.0) * (1.0 / 4294967296.0);
        double u2 = (double)w[1] * (1.0 / 4294967296.0);
        double uu = ((double)w[2] + 1.0) * (1.0 / 4294967296.0);
        double z = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
        double t = 1.0 + c * z;
        *margin = min2(*margin, fabs(t));
        if (t <= 0.0)
            continue;
        double v = t * t * t;
        double lhs = log(uu);
        double rhs = 0.5 * z * z + d - d * v + d * log(v);
        *margin = min2(*margin, fabs(lhs - rhs) / scale);
        if (lhs < rhs)
            return d * v;
    }
    return d;
}

/* Beta(a, b) = X / (X + Y) with X ~ Gamma(a), Y ~ Gamma(b), both shapes >= 1. */
double oracle_beta_sample(double a, double b, uint64_t seed, uint64_t offset, int group,
                          int arm, double *margin)
{
    double x = oracle_gamma_mt(a, seed, offset, group, arm, 0, margin);
    double y = oracle_gamma_mt(b, seed, offset, group, arm, 1, margin);
    return x / (x + y);
}

/* Relative gap between the best and the runner-up of K scores (+inf if K == 1). */
static double top_gap(const double *score, int K, int best)
{
    double gap = INFINITY;
    for (int j = 0; j < K; ++j) {
        if (j == best)
            continue;
        double g = (score[best] - score[j]) / fabs(score[best]);
        gap = min2(gap, g);
    }
    return gap;
}

/* First index of the largest score (B4). */
static int argmax_first(const double *score, int K)
{
    int best = 0;
    for (int j = 1; j < K; ++j)
        if (score[j] > score[best])
            best = j;
    return best;
}

/*
 * UCB1 for one group: any arm not yet played is played first, lowest index
 * first; otherwise the index mean_j + sqrt(2 ln n / n_j) decides.
 */
int oracle_ucb1_select(int K, const uint32_t *counts, const double *sums, double *margin)
{
    uint64_t n = 0;
    for (int j = 0; j < K; ++j) {
        if (counts[j] == 0) {
            *margin = INFINITY;
            return j;
        }
        n += counts[j];
    }
    double score[BANDIT_MAX_ARMS];
    for (int j = 0; j < K; ++j) {
        double nj = (double)counts[j];
        double mean = sums[j] / nj;
        double bonus = sqrt(2.0 * log((double)n) / nj);
        score[j] = mean + bonus;
    }
    int best = argmax_first(score, K);
    *margin = top_gap(score, K, best);
    return best;
}

/* Thompson sampling for one group: theta_j ~ Beta(1 + S_j, 1 + n_j - S_j). */
int oracle_thompson_select(int K, const uint32_t *counts, const double *sums,
                           uint64_t seed, uint64_t offset, int group, double *margin)
{
    double theta[BANDIT_MAX_ARMS];
    *margin = INFINITY;
    for (int j = 0; j < K; ++j) {
        double a = 1.0 + sums[j];
        double b = 1.0 + ((double)counts[j] - sums[j]);
        theta[j] = oracle_beta_sample(a, b, seed, offset, group, j, margin);
    }
    int best = argmax_first(theta, K);
    *margin = min2(*margin, top_gap(theta, K, best));
    return best;
}

/*
 * One round for every group: fold in the accept lengths of the last
 * verification (if accept_len is not NULL) for the arm each group played,
 * then choose each group's next arm. counts/sums are [G][K] and updated in
 * place; out_arm and out_margin are [G].
 */
void oracle_bandit_step(int policy, int G, int K, int B, int gamma,
                        uint32_t *counts, double *sums,
                        const int32_t *accept_len, const int32_t *arm_played,
                        uint64_t seed, uint64_t offset,
                        int32_t *out_arm, double *out_margin)
{
    const int per = B / G;
    for (int g = 0; g < G; ++g) {
        uint32_t *cg = counts + (size_t)g * K;
        double *sg = sums + (size_t)g * K;
        if (accept_len) {
            int a = arm_played[g];
            if (a < 0 || a >= K) {
                out_arm[g] = -1;
                out_margin[g] = INFINITY;
                continue;
            }
            int64_t ksum = 0;
            int64_t m = 0;
            for (int b = g * per; b < (g + 1) * per; ++b) {
                int k = accept_len[b];
                if (k >= 0 && k <= gamma) {
                    ksum += k;
                    m += 1;
                }
            }
            if (m > 0) {
                double r = (double)ksum / ((double)gamma * (double)m);
                cg[a] += 1;
                sg[a] += r;
            }
        }
        if (policy == BANDIT_UCB1)
            out_arm[g] = oracle_ucb1_select(K, cg, sg, &out_margin[g]);
        else
            out_arm[g] = oracle_thompson_select(K, cg, sg, seed, offset, g, &out_margin[g]);
    }
}
