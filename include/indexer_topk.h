/*
 * indexer_topk.h -- C ABI of the MI355X (gfx950) indexer scoring and the
 * fused scoring + exact top-k (the step before the top-k + transform).
 *
 * The operation is the DSA indexer of a prefill batch as LiteTopk PR #32094
 * "Add LiteTopk fused indexer top-k prefill path for SM100" defines it
 * (Summary; Background list: score, gate, compact exact select; Validation:
 * the reference formula):
 *
 *   score[r, j] = kv_scale[j] * sum_h weights[r, h] * relu(q[r, h, :] . kv[j, :])
 *
 * for the positions j of row r's key range [ks[r], ke[r]), with H = 32 heads
 * of D = 128 (the GLM indexer shape the page is restricted to).  q and kv are
 * fp8 E4M3 codes (OCP encoding: bias 7, no infinities, 0x7F / 0xFF are NaN;
 * NaN codes are outside the contract).  The library widens them exactly and
 * sums in fp32, so every score is within a few fp32 rounding errors of the
 * exact value: |fp32 - exact| <= (D + H + 2) * 2^-24 * kv_scale[j] *
 * sum_h |weights[r, h]| * sum_d |q[r, h, d] * kv[j, d]| (to first order).
 *
 * Both calls share topk_transform.h's status codes, topk_last_error() and
 * topk_release_workspaces().
 */
#ifndef INDEXER_TOPK_H_
#define INDEXER_TOPK_H_

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "topk_transform.h"

#ifdef __cplusplus
extern "C" {
#endif

#define INDEXER_HEADS 32
#define INDEXER_HEAD_DIM 128

/*
 * indexer_logits -- the dense scores (what the fused call avoids writing).
 *
 *   q          (num_q, 32, 128) uint8 fp8 codes, row-major.  Read only.
 *   weights    (num_q, 32) fp32.  Read only.
 *   kv         (num_kv, 128) uint8 fp8 codes, row-major; 16-byte aligned.
 *   kv_scale   (num_kv,) fp32.
 *   ks, ke     (num_q,) int32: row r's key range [ks[r], ke[r]), each clamped
 *              to [0, num_kv]; an empty or inverted range is an empty row.
 *   logits     (num_q, logits_stride) fp32, written: logits[r, c] is the
 *              score of position ks[r] + c for c < min(ke[r] - ks[r],
 *              logits_stride).  Other entries are left untouched.
 *   stream     HIP stream the work is queued on.
 *   num_q      rows, >= 0 (0 is a no-op).  num_kv >= 0.  logits_stride >= 0.
 *
 * All pointers are device pointers on the current device; the caller owns
 * them and the library keeps none past the call.  Asynchronous on `stream`.
 * Errors: TOPK_ERROR_INVALID_VALUE (null pointer with num_q > 0 or a negative
 * size, kv not 16-byte aligned), TOPK_ERROR_UNSUPPORTED (device not gfx950),
 * TOPK_ERROR_LAUNCH.  On error nothing was queued.
 */
topk_status_t indexer_logits(const uint8_t* q, const float* weights, const uint8_t* kv, const float* kv_scale,
                             const int32_t* ks, const int32_t* ke, float* logits, hipStream_t stream,
                             int32_t num_q, int64_t num_kv, int64_t logits_stride);

/*
 * indexer_topk -- fused scoring + exact top-k over each row's key range,
 * without a dense [num_q, length] score buffer (LiteTopk PR #32094, Summary
 * and Background: the scan keeps only positions that pass a gate that only
 * tightens; the select trims the survivors exactly).
 *
 *   q, weights, kv, kv_scale, ks, ke   as in indexer_logits.
 *   k          1 <= k <= TOPK_MAX_K.
 *   out_idx    (num_q, k) int32, written.  Slots [0, n_r), n_r =
 *              min(k, ke[r] - ks[r]) (after clamping), hold n_r distinct
 *              absolute key positions of the range that form a top-n_r set of
 *              the row's fp32 scores (as computed by indexer_logits, ties at
 *              the cut filled by any equal-score positions); slots [n_r, k)
 *              hold -1 (LiteTopk PR, "sglang deviations": -1 padding, output
 *              coordinates are absolute positions in the gathered key buffer).
 *              The order within [0, n_r) is unspecified.
 *   stream, num_q, num_kv              as in indexer_logits.
 *
 * Two internal forms, same result contract.  Where each workgroup's window
 * of key positions is long against k (window >= 64 k), or the score buffer
 * would exceed 8 GiB, the fused scan keeps gated candidate lists and the
 * exact top-k of the candidates runs through topk_transform on the same
 * stream.  On shorter windows every window keeps a large share of its
 * positions, and the list work costs more than writing every score: those
 * calls score densely into a buffer and select from it with topk_transform
 * (indexer_set_select_mode forces either form).
 * Working memory: per (device, stream), the fused form's candidate lists of
 * num_q x windows x max(4k, 4096) (score, position) pairs plus num_q x
 * windows x k packed candidates, or the dense form's num_q x num_kv scores
 * plus num_q x (k + 1) words, allocated on first need, grown on demand (a
 * replaced buffer stays allocated, so graphs captured with it stay valid) and
 * freed by topk_release_workspaces().
 * Errors: as indexer_logits, plus TOPK_ERROR_INVALID_VALUE for k outside
 * [1, TOPK_MAX_K] and TOPK_ERROR_OUT_OF_MEMORY.
 */
topk_status_t indexer_topk(const uint8_t* q, const float* weights, const uint8_t* kv, const float* kv_scale,
                           const int32_t* ks, const int32_t* ke, int32_t k, int32_t* out_idx, hipStream_t stream,
                           int32_t num_q, int64_t num_kv);

/*
 * Testing and tuning override, process-wide: the number of key positions each
 * workgroup's window covers (the key range is split into windows so that
 * short batches still fill the device).  0 = automatic; otherwise a positive
 * multiple of 64.  Any window gives the same result; the choice only moves
 * time and how often the candidate lists are trimmed.
 * Returns TOPK_ERROR_INVALID_VALUE for other values.
 */
topk_status_t indexer_set_window_override(int64_t window);

/*
 * Testing and tuning override of indexer_topk's internal form, process-wide:
 * -1 automatic (the default: dense when the window is shorter than 64 k and
 * the score buffer fits 8 GiB), 0
 * the fused scan, 1 dense scores + select.  Both give a result that meets
 * indexer_topk's contract; the choice only moves time and working memory.
 * Returns TOPK_ERROR_INVALID_VALUE for other values.
 */
topk_status_t indexer_set_select_mode(int32_t mode);

#ifdef __cplusplus
}
#endif

#endif /* INDEXER_TOPK_H_ */
