/*
 * spec_head.h -- C ABI of the low-rank draft LM head with its fused row
 * normaliser, on AMD Instinct MI355X (gfx950).
 *
 * The operation (SlimSpec summary, Methodology, architecture): the draft's LM
 * head z = W_full h, W_full in R^{V x d}, is factored as z = W_up W_down h with
 * W_down in R^{r x d}, W_up in R^{V x r} and r << d, computed with dense matrix
 * products, which cuts the head from O(Vd) to O(rd + Vr). Its logits are the
 * draft rows the verifier reads, so the head also returns each row's
 * log-normaliser, produced while the logits are still on chip instead of by a
 * second pass over them.
 *
 * Precise definition, per row n with T = temperature[n]:
 *   u = bf16(W_down h_n)           (rank-r activation, rounded to nearest even)
 *   z = bf16(W_up u)               (V logits, rounded to nearest even)
 *   lse[n] = log sum_v exp(fl32(z_v * fl32(1/T)))   for T > 0 (NaN otherwise),
 * the normaliser the verifier computes for a draft row. The products are
 * accumulated in binary32 on the matrix cores (each product of two bf16
 * values is exact in binary32); the results equal the exact values' roundings
 * except where an exact value lies within the binary32 accumulation error of
 * a bf16 rounding boundary.
 *
 * Layouts: dense row-major bf16 (uint16 bit patterns) device arrays
 *   hidden [N, d], w_down [r, d], w_up [V, r], out_logits [N, V];
 *   temperature [N] float32, out_lse [N] float64.
 * Requirements: d % 64 == 0, r % 64 == 0, V % 8 == 0, every bf16 array 16-byte
 * aligned (SPEC_EINVAL otherwise). All pointers are DEVICE pointers owned by
 * the caller; the library owns only its workspace (about 2 N r bytes plus
 * N * V / 8 bytes).
 *
 * Asynchrony and errors: as in spec_verify.h. spec_lowrank_head enqueues three
 * kernels on the context's stream and returns.
 */
#ifndef SPEC_HEAD_H
#define SPEC_HEAD_H

#include <stdint.h>

#include "spec_verify.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct spec_head_ctx spec_head_ctx;

/* Workspace for heads of this shape; hip_stream may be NULL (null stream). */
int spec_lowrank_head_init(int rows, int hidden, int rank, int vocab, void* hip_stream,
                           spec_head_ctx** out_ctx);

int spec_lowrank_head_set_stream(spec_head_ctx* ctx, void* hip_stream);

/* Logits and row log-normalisers of the draft rows (definition above). */
int spec_lowrank_head(spec_head_ctx* ctx, const void* hidden, const void* w_down,
                      const void* w_up, const float* temperature, void* out_logits,
                      double* out_lse);

/* Test hook: the rank-r activation u [N, r] (bf16) of the last call, copied
 * to the device array out_u on the context's stream. */
int spec_lowrank_head_copy_activation(spec_head_ctx* ctx, void* out_u);

int spec_lowrank_head_destroy(spec_head_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_HEAD_H */
