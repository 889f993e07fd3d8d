/*
 * spec_bandit.h -- C ABI of online draft-model selection on the device.
 *
 * The operation (FlashSpec technical summary, Methodology section 2, "draft
 * selection via online bandit"): choosing which of K draft models proposes
 * the next gamma tokens is a K-armed bandit; the reward of a play is the
 * fraction of draft tokens the verifier accepted, and the policy is UCB1 or
 * Thompson sampling. Because the choice looks only at past accept counts, the
 * verified output keeps the target's distribution (same summary, Significance
 * section, Theorem 1). Keeping the bandit on the device lets it read the
 * verifier's out_accept_len where it lies, with no host round trip.
 *
 * Precise definition. Sequences are split into G groups of B/G consecutive
 * sequences; each group is one independent bandit (G = 1: one arm per step
 * for the whole batch; G = B: one bandit per sequence slot). Its state is, per
 * arm j, the play count n_j (uint32) and the reward sum S_j (double).
 * A step, per group g:
 *   1. (when accept_len is given) with a = arm_played[g] and the m
 *      sequences b of the group whose accept_len[b] lies in [0, gamma]:
 *      if m > 0, n_a += 1 and S_a += (sum_b accept_len[b]) / (gamma * m)
 *      (one double division, correctly rounded); if m == 0 nothing changes;
 *   2. the next arm:
 *      UCB1 (Auer, Cesa-Bianchi and Fischer, Machine Learning 47, 2002,
 *      Fig. 1): the lowest-index arm with n_j == 0 if any, else the arm
 *      maximising S_j / n_j + sqrt(2 ln n / n_j), n = sum_j n_j;
 *      Thompson sampling (Agrawal and Goyal, COLT 2012) with a Beta(1, 1)
 *      prior: the arm maximising theta_j ~ Beta(1 + S_j, 1 + n_j - S_j),
 *      Beta = X / (X + Y) of two Gamma variates drawn by Marsaglia and Tsang
 *      (ACM TOMS 26(3), 2000, no squeeze step, at most 64 attempts, then the
 *      variate is shape - 1/3) from Box-Muller normals (cosine branch).
 *      Ties go to the lowest index. Everything is IEEE double.
 *   Uniforms: Philox4x32-10 with key (lo32(seed), hi32(seed)) and counter
 *   (2^31 | (64 (2 j + s) + attempt), g, lo32(offset), hi32(offset)), s = 0 for
 *   X and 1 for Y; u1 = (w0 + 1) 2^-32, u2 = w1 2^-32, U = (w2 + 1) 2^-32. The
 *   set top bit keeps these counters apart from spec_verify's, so the same
 *   (seed, offset) may be given to both.
 *
 * Layouts: accept_len [B], arm_played [G] and out_arm [G] are int32 DEVICE
 * arrays owned by the caller; out_arm may be the same array as arm_played.
 * The library owns the state (G * K * 12 bytes of device memory).
 *
 * Asynchrony: spec_bandit_step enqueues one kernel on the context's stream
 * and returns. spec_bandit_get_state / spec_bandit_set_state synchronise
 * that stream. A context is not thread-safe.
 *
 * Errors: the status codes of spec_verify.h. Host-detectable problems (NULL
 * context or pointer, bad sizes, misaligned pointer) return SPEC_EINVAL before
 * any launch; a failed launch returns SPEC_EHIP. Bad DATA is handled on the
 * device: accept lengths outside [0, gamma] are left out of the reward, and a
 * group whose arm_played lies outside [0, K) is not updated and gets
 * out_arm[g] = -1.
 */
#ifndef SPEC_BANDIT_H
#define SPEC_BANDIT_H

#include <stdint.h>

#include "spec_verify.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct spec_bandit_ctx spec_bandit_ctx;

enum { SPEC_BANDIT_UCB1 = 0, SPEC_BANDIT_THOMPSON = 1 };

/* Largest number of arms (one wavefront lane per arm). */
#define SPEC_BANDIT_MAX_ARMS 64

/*
 * Create G bandits of K arms (1 <= K <= 64) over B sequences (B % G == 0)
 * verified with gamma >= 1 draft tokens; policy is SPEC_BANDIT_UCB1 or
 * SPEC_BANDIT_THOMPSON. hip_stream (a hipStream_t, may be NULL for the null
 * stream) is where steps run. The state starts at zero (no plays).
 */
int spec_bandit_init(int n_groups, int n_arms, int batch, int gamma, int policy,
                     void* hip_stream, spec_bandit_ctx** out_ctx);

/* Move later steps to another stream. */
int spec_bandit_set_stream(spec_bandit_ctx* ctx, void* hip_stream);

/*
 * One round for every group: fold in accept_len [B] for the arms the groups
 * played (arm_played [G]), then write each group's next arm to out_arm [G].
 * With accept_len == NULL only the choice is made (arm_played is ignored and
 * may be NULL), as for the very first step. seed and offset pick the Thompson
 * draws (UCB1 uses none); advance offset by one per step.
 */
int spec_bandit_step(spec_bandit_ctx* ctx, const int32_t* accept_len, const int32_t* arm_played,
                     uint64_t seed, uint64_t offset, int32_t* out_arm);

/* Copy the state to HOST arrays counts [G*K] and sums [G*K] (group-major). */
int spec_bandit_get_state(spec_bandit_ctx* ctx, uint32_t* counts, double* sums);

/*
 * Overwrite the state from HOST arrays counts [G*K] and sums [G*K], e.g. to
 * resume from a saved state; both NULL resets it to zero. Each sums entry must
 * lie in [0, counts entry]; otherwise SPEC_EINVAL and nothing changes.
 */
int spec_bandit_set_state(spec_bandit_ctx* ctx, const uint32_t* counts, const double* sums);

/* Wait for the context's stream, free the state and the context. */
int spec_bandit_destroy(spec_bandit_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_BANDIT_H */
