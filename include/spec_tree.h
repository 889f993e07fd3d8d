/*
 * spec_tree.h -- C ABI for draft trees on AMD Instinct MI355X (gfx950):
 * confidence-guided pruning, and greedy and sampled tree verification.
 *
 * Pruning (SpecLA summary, Methodology section 3, target-aligned drafting):
 * low-probability paths of a draft tree are cut by their cumulative draft
 * log-probability before the target verifies them. Tree b has M nodes in
 * topological order: node 0 is the root (the last verified token) and node
 * i >= 1 hangs under parent[i] in [0, i), carrying logq[i] <= 0, its draft
 * token's log-probability given its path. Definition:
 *   c(0) = 0, c(i) = c(parent(i)) + (double)logq(i), summed from the root down;
 *   node i is kept iff c(i) >= tau and fewer than `budget` nodes have a larger
 *   c (ties to the lower index). Scores never rise along a path, so the kept
 *   set contains every kept node's ancestors; kept nodes are renumbered in
 *   index order.
 * A tree whose parent array is not topological or with a NaN or positive
 * logq is a sentinel: count -1, nothing kept, scores NaN.
 *
 * Greedy verification (T = 0; the exact-match rule of token-tree speculative
 * decoding, Miao et al., SpecInfer, ASPLOS 2024; on a chain it is
 * spec_verify's greedy rule): the target's logits are given for every node,
 * row i holding the distribution of the token after node i's path; a(i) is
 * its argmax over raw logits (lowest index on ties). From the root the walk
 * steps to the lowest-index child whose token is a(x), while there is one;
 * the result is the accepted nodes, their count, and the extra token a(last).
 * Trees with n_nodes outside [1, M], a parent outside [0, i), a token outside
 * [0, V), or a reached row with no finite logit get length -1, path -1 and
 * extra token -1.
 *
 * Sampled verification (T > 0): multi-step speculative sampling (Miao et al.,
 * SpecInfer, ASPLOS 2024, stochastic tree verification), the published
 * multi-branch rule that keeps the target's output distribution when the
 * children of node u are draft tokens drawn independently from q_u. The
 * pages name tree drafting but give no such rule. Draft row u is q_u, target
 * row u is p_u (both as the verifier scales them, x = fl32(z * fl32(1/T))).
 * At node u with current target pi (pi = p_u on arrival), u's children are
 * tried in increasing node order: child s with token t is accepted iff
 * log u_acc < log pi(t) - log q_u(t) (fp64), and the walk moves to s;
 * otherwise pi <- norm(max(0, pi - q_u)) (kept when that mass is zero, which
 * only rounding produces) and the next child is tried. When u has no child
 * left, the extra token is drawn from pi by inversion in vocabulary order.
 * Uniforms: Philox4x32-10 as in spec_verify.h, block (s - 1, b) word 0 for
 * child s, block (L, b) word 1 for the draw (L accepted nodes), so a chain
 * (node i + 1 holding draft token i) sees the verifier's uniforms and gives
 * its outcome. T == 0 trees follow the greedy rule above; invalid
 * temperatures are sentinels as in spec_verify.h. Outputs as for the greedy
 * call. Cost: one pass over the two rows of each visited node with children
 * (the target row alone at a leaf), one per rejection, one for the draw when
 * the last node rejected nothing. Each tree is split over four 256-thread
 * workgroups that own quarters of the vocabulary and exchange per-pass
 * results through the context's workspace; the launch holds at most as many
 * trees as the device keeps resident at once (the rest follow in turn), and
 * calls on one context must not overlap. The exchange tags each launch with a
 * launch number that the kernel keeps in the context's workspace, so the call
 * may be captured into a HIP graph and replayed. A part that waits about a
 * second for a partner (possible only if other work keeps the partner off the
 * device) gives up; part 0 then reports that tree and the later trees of its
 * group with length -2 (distinct from the -1 of invalid input), path and extra
 * token -1, and adds them to a count that spec_tree_verify_gave_up reads.
 *
 * Layouts: dense row-major DEVICE arrays owned by the caller; int32 indices,
 * float32 logq, float64 scores; target logits [B, M, V] in the dtype of
 * spec_verify.h (16-byte-aligned rows take the vector path). 1 <= M <=
 * SPEC_TREE_MAX_NODES. Calls enqueue kernels on the given (or context's)
 * stream and return; host-detectable errors return SPEC_EINVAL first.
 */
#ifndef SPEC_TREE_H
#define SPEC_TREE_H

#include <stdint.h>

#include "spec_verify.h"

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_TREE_MAX_NODES 256

/* Prune B trees of M nodes. Outputs: out_cum [B, M] float64, out_new_index
 * [B, M] (new position or -1), out_new_parent [B, M] (by new position, -1 for
 * the root and unused slots), out_count [B]. No workspace; hip_stream may be
 * NULL. */
int spec_tree_prune(int batch, int nodes, const int32_t* parent, const float* logq, double tau,
                    int budget, double* out_cum, int32_t* out_new_index,
                    int32_t* out_new_parent, int32_t* out_count, void* hip_stream);

typedef struct spec_tree_ctx spec_tree_ctx;

/* Workspace for verification of B trees of at most M nodes over a
 * vocabulary of V logits of the given dtype (greedy: per-split argmax
 * results; sampled: the parts' exchange slots, zeroed here). */
int spec_tree_verify_init(int batch, int max_nodes, int vocab, int dtype, void* hip_stream,
                          spec_tree_ctx** out_ctx);

int spec_tree_verify_set_stream(spec_tree_ctx* ctx, void* hip_stream);

/* parent, token [B, M] int32 (token[b][0] ignored), n_nodes [B], target
 * [B, M, V]; outputs out_length [B], out_path [B, M] (accepted node indices in
 * order, -1 padded), out_extra [B]. Rows of nodes >= n_nodes are not read. */
int spec_tree_verify_greedy(spec_tree_ctx* ctx, const int32_t* parent, const int32_t* token,
                            const int32_t* n_nodes, const void* target, int32_t* out_length,
                            int32_t* out_path, int32_t* out_extra);

/* draft, target [B, M, V] in the context's dtype (draft row u: the
 * distribution u's children were drawn from), temperature [B] fp32, seed and
 * offset as in spec_verify.h; other arguments and outputs as for
 * spec_tree_verify_greedy. Uses the context's workspace; SPEC_EINVAL when V
 * exceeds the 16 KiB of tile sums one part keeps in LDS (V > 1 048 576) or
 * ceil(B / resident trees) * (2M + 2) >= 2^20. */
int spec_tree_verify_sample(spec_tree_ctx* ctx, const int32_t* parent, const int32_t* token,
                            const int32_t* n_nodes, const void* draft, const void* target,
                            const float* temperature, uint64_t seed, uint64_t offset,
                            int32_t* out_length, int32_t* out_path, int32_t* out_extra);

/* Number of trees reported with length -2 (a part gave up waiting for a
 * partner) by all sampled calls on this context so far. Synchronises the
 * context's stream. */
int spec_tree_verify_gave_up(spec_tree_ctx* ctx, uint64_t* out_count);

/* Test hook: the polls a part makes before giving up on a partner (default
 * 2^20, about a second). A small value makes the bounded wait give up from
 * the host side while every kernel still exits normally. polls >= 0. */
int spec_tree_verify_set_spin_limit(spec_tree_ctx* ctx, int polls);

int spec_tree_verify_destroy(spec_tree_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_TREE_H */
