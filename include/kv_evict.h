/*
 * kv_evict.h — budgeted KV eviction selection on the GPU (part of libkvattn.so).
 *
 * What is computed (Ch. 19 "Inference Systems and Performance Engineering", §19.4.3, the
 * programming exercise on eviction under a global memory budget): every (layer l, KV head h,
 * position t) entry of the cache carries an attention score, and at most M entries may stay.
 *   1. The current position C of every (layer, head) row stays unconditionally; that costs L*H
 *      of the budget.
 *   2. All other entries compete in one pool, regardless of layer or head, so different layers
 *      can end up keeping different numbers of tokens.
 *   3. The pool is ranked by the key (-score, l, h, t) in ascending order: larger scores first,
 *      equal scores by layer, then head, then position, each ascending.
 *   4. The first M - L*H entries of that ranking stay. The key is a total order, so the kept
 *      set is unique.
 * The page ranks the pool with one global sort. Here the same set comes from a radix selection
 * of the (M - L*H)-th largest 64-bit key (score bits made order-preserving, then the complement
 * of the flat index (l*H + h)*N + t, so that ties fall to the lower index): a sample of the
 * scores places a narrow band of key values around that key, one streaming pass over the scores
 * writes the mask outside the band and sets the band's entries aside while counting exactly,
 * and passes over the set-aside entries finish the selection. Should the exact counts show that
 * the selected key lies outside the band (a sample unlike the rest of the scores), one workgroup
 * computes the whole selection exactly instead: the result is the same, only slower.
 *
 * Readings where the page is silent: scores compare as values (-0.0 ties with +0.0, +-inf are
 * allowed, NaN is outside the contract); C is one position shared by every row; when
 * M <= L*H only the current positions stay, and when M - L*H covers the whole pool everything
 * stays.
 */
#ifndef KV_EVICT_H_
#define KV_EVICT_H_

#include <stddef.h>
#include <stdint.h>

#include "kv_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kv_evict_params {
  int32_t num_layers;  /* L >= 1 */
  int32_t num_heads;   /* H >= 1: KV heads, the unit whose entries stay or go */
  int32_t num_tokens;  /* N >= 1 positions per (layer, head) row; L * H * N < 2^31 */
  int32_t current;     /* C, 0 <= C < N: the current position, kept in every row */
  int64_t budget;      /* M >= 0: entries that may stay in total */
  int64_t row_stride;  /* elements between consecutive rows of `scores` (>= N) */
} kv_evict_params;

/*
 * Workspace bytes kv_evict_select needs for `p`: 0 when the budget alone decides the result
 * (M - L*H <= 0, or M - L*H >= L*H*(N - 1)), otherwise 930048 bytes of selection state and
 * histograms plus two candidate lists of 8 bytes per slot, each with at least L*H*N slots
 * (rounded up to whole blocks of 16384 entries per workgroup). Returns 0 for invalid `p`.
 */
size_t kv_evict_workspace_size(const kv_evict_params* p);

/*
 * Select the entries that stay (rules 1-4 above).
 *
 * scores       : device fp32; row r = l*H + h holds positions 0..N-1 at scores + r*row_stride.
 *                4-byte aligned. Only read. NaN values are outside the contract (they rank
 *                deterministically but meaninglessly).
 * keep         : device uint8 [L*H, N] contiguous, written in full: 1 where the entry stays,
 *                0 where it is evicted. Must not alias scores or the workspace.
 * kept_per_row : device int32 [L*H] receiving the number of entries that stay in each row, or
 *                NULL.
 * workspace    : device scratch of at least kv_evict_workspace_size(p) bytes, 16-byte aligned
 *                (NULL allowed when that size is 0); contents need no initialisation and are
 *                left unspecified.
 * stream       : hipStream_t (NULL = default stream); every kernel is enqueued there and the
 *                call returns without synchronising. Calls that share a workspace must not
 *                overlap.
 * Returns KV_ATTN_ERR_NULL (scores, keep or p missing), KV_ATTN_ERR_SHAPE (a size < 1, C out of
 * range, row_stride < N), KV_ATTN_ERR_VALUE (budget < 0), KV_ATTN_ERR_UNSUPPORTED (L*H*N >=
 * 2^31, misaligned pointers), KV_ATTN_ERR_WORKSPACE, all before anything is launched, or
 * KV_ATTN_ERR_HIP if a launch fails.
 * Environment: KV_EVICT_FORCE_FALLBACK=1 (read at each call; a test aid) sends every ranked call
 * down the exact single-workgroup path; the mask is the same.
 */
kv_attn_status kv_evict_select(const float* scores, uint8_t* keep, int32_t* kept_per_row,
                               const kv_evict_params* p, void* workspace, size_t workspace_bytes,
                               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KV_EVICT_H_ */
