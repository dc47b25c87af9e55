/*
 * pa_sample.h -- batched token sampling over the logits rows of one tick:
 * greedy, temperature, top-k and top-p, every row with its own settings, all
 * rows in one launch.
 *
 * What it follows: the sampler offers greedy, temperature, top-k and top-p
 * (llm-serving-engine README, component table row "Token sampling");
 * temperature lies in [0, 2] and top-p in (0, 1] (Helios README, the request
 * fields); rows are sampled together rather than one by one (Helios blog,
 * "Continuous batching"), and batched sampling equals sampling each row alone
 * (mini-vLLM page, "Test suites").
 *
 * The definition, per row r with logits x[0 .. V), temperature T, top_k k,
 * top_p p and the caller's uniform u in [0, 1):
 *   - T <= 0 (or NaN), or k == 1: greedy, the index of the largest logit (the
 *     lowest index among equal ones).
 *   - Ranking: larger logit first, equal logits (-0.0 with +0.0) by lower index.
 *   - Weights: w_i = floor(exp((x_i - max) / T) * 2^32), computed in float64
 *     (IEEE subtraction and division, then exp), held as exact integers.
 *   - Top-k keeps the first k of the ranking (k <= 0 or k >= V: all). Top-p
 *     then keeps the shortest leading part of that whose total weight reaches
 *     ceil(p * S_k), S_k the total weight top-k kept (p >= 1: all; p <= 0:
 *     the first token).
 *   - The token is the first index, in index order among the kept tokens, at
 *     which the running weight exceeds floor(u * S), S the kept total.
 * Logits must be finite or -inf, with a finite maximum; anything else yields
 * some index in [0, V) and no fault.
 *
 * All pointers are device memory. logits: float32 [rows, row_stride], the
 * first vocab entries of each row used. temperature, top_p, uniforms: float32
 * [rows]; top_k: int32 [rows]; out_tokens: int32 [rows], written. rows >= 0
 * (0 enqueues nothing); 1 <= vocab <= 2^21 (else PA_ERR_UNSUPPORTED);
 * row_stride >= vocab; rows * ceil(vocab / 3072) <= 2^30. workspace: device memory
 * of at least pa_sample_workspace_size(rows, vocab) bytes, 256-byte aligned, owned by the caller,
 * used only while the call's kernels run (calls that share one workspace must
 * not overlap); it needs no clearing. PA_ERR_INVALID_ARG for a bad scalar, a
 * NULL pointer (when rows > 0) or a misaligned workspace,
 * PA_ERR_WORKSPACE_TOO_SMALL for a short one; nothing is enqueued then.
 * Asynchronous on `stream` (a hipStream_t; NULL = the default stream): two
 * launches, a screen of 3072-token slices of the rows, then one workgroup per
 * row.
 */
#ifndef PA_SAMPLE_H
#define PA_SAMPLE_H

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workspace bytes pa_sample_tokens needs for `rows` rows of `vocab` logits
 * (0 for rows <= 0 or a vocab outside [1, 2^21]). */
size_t pa_sample_workspace_size(int32_t rows, int32_t vocab);

pa_status_t pa_sample_tokens(const float* logits, int64_t row_stride, int32_t rows,
                             int32_t vocab, const float* temperature, const int32_t* top_k,
                             const float* top_p, const float* uniforms, int32_t* out_tokens,
                             void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_SAMPLE_H */
