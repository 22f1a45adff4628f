/*
 * loss.h — C ABI of the fused loss kernels for MI355X (gfx950).
 *
 * The operations of the page "cross_entropy ve sum_losses — Fused Loss +
 * dLogits" (https://llm.istanbul/learn/tr/07_loss), sections "Ne Yapar?" and
 * "Satır Satır": for every row s of the lm_head logits [S x V],
 *
 *   lse      = max_v l[v] + log(max(sum_v exp(l[v] - max), 1e-30))
 *   p[v]     = exp(l[v] - max) / max(sum, 1e-30)
 *   loss[s]  = lse - (1 - alpha) l[tgt] - alpha mean_v l[v] + beta lse^2
 *   dl[v]    = ((p[v] - target[v]) + 2 beta lse p[v]) * inv_norm,
 *              target = (1 - alpha) one_hot(tgt) + alpha / V
 *
 * with label smoothing alpha and z-loss beta; the gradient overwrites the
 * logits in place.  A row whose target is >= V (padding) gets loss 0 and an
 * all-zero gradient row.  sum_losses adds the S per-row losses.
 *
 * Layout: logits [S x V] fp32 row-major, targets [S] uint32, losses [S] fp32,
 * out [1] fp32; all device pointers owned by the caller.  A call only
 * enqueues work on `stream` (a hipStream_t, NULL for the null stream).  Each
 * row is reduced in a fixed order, so results are bitwise reproducible.
 *
 * Errors are returned synchronously, before anything is enqueued (the status
 * values are those of gemm_fwd.h): GEMM_ERR_NULL for a missing array,
 * GEMM_ERR_SHAPE for S < 0, V < 0, S >= 2^31 or V >= 2^29, GEMM_ERR_ALIGN for
 * an array not 4-byte aligned, GEMM_ERR_DTYPE for alpha outside [0, 1], a
 * negative or non-finite beta or a non-finite inv_norm, GEMM_ERR_ALIAS when
 * losses overlaps logits or targets (or out overlaps losses), and
 * GEMM_ERR_LAUNCH when the runtime rejects the launch.
 */
#ifndef LOSS_H
#define LOSS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * cross_entropy: losses[s] and the in-place gradient of every row.
 * S == 0 enqueues nothing; V == 0 makes every row an ignored row.
 */
int loss_cross_entropy(float *logits, const uint32_t *targets, float *losses, int64_t S, int64_t V,
                       float alpha, float beta, float inv_norm, void *stream);

/* sum_losses: out[0] = sum of losses[0 .. S-1] (0 when S == 0), one workgroup. */
int loss_sum_losses(const float *losses, float *out, int64_t S, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LOSS_H */
