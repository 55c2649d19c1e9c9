/*
 * topk_transform.h -- C ABI of the MI355X (gfx950) fused top-k + page-table transform.
 *
 * The operation is the sparse-attention indexer's per-row selection step: for
 * each row of fp32 index scores, pick the k positions with the greatest scores
 * among the row's first seq_len entries, and map each selected position through
 * that row's KV page table.  It is the operation of SGLang PR #26788
 * "DeepSeek-V4 DSA indexer: faster top-k + page-table transform (runtime
 * k <= 2048)" (Motivation and Feature sections: runtime k up to 2048, ragged
 * per-row sequence lengths, arbitrary power-of-two page size, optional raw
 * pre-transform index output), implemented from scratch for CDNA4.
 *
 * Every function is a plain C call: pointers, sizes and a HIP stream.  No
 * exception crosses this boundary; every failure is a status code.
 */
#ifndef TOPK_TRANSFORM_H_
#define TOPK_TRANSFORM_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest k accepted (PR #26788 title and Feature section: runtime k <= 2048). */
#define TOPK_MAX_K 2048

typedef enum topk_status_t {
  TOPK_SUCCESS = 0,
  /* A required pointer is NULL (seq_lens and out_idx always; scores when
   * width > 0; page_table when pages_per_row > 0), k is outside
   * [1, TOPK_MAX_K], page_size is not a power of two, batch / width /
   * pages_per_row is negative, or width exceeds INT32_MAX. */
  TOPK_ERROR_INVALID_VALUE = 1,
  /* The current device is not gfx950, or the shape needs more cooperating
   * workgroups than the device can hold resident at once. */
  TOPK_ERROR_UNSUPPORTED = 2,
  /* The internal workspace could not be allocated. */
  TOPK_ERROR_OUT_OF_MEMORY = 3,
  /* A HIP call failed; topk_last_error() holds the HIP error text. */
  TOPK_ERROR_LAUNCH = 4,
  /* An earlier split-row launch queued on the same stream gave up one of its
   * bounded cross-workgroup waits (its workgroups were not all resident at
   * once, e.g. because another kernel held CUs), so that launch's outputs
   * are invalid and must be recomputed.  Reported once, by the next call on
   * that stream that sees it or by topk_check_faults; the reporting call
   * queued nothing.  The launch that gave up put the workspace back in its
   * initial state, so calls after the report run normally. */
  TOPK_ERROR_DEVICE_FAULT = 5
} topk_status_t;

/*
 * topk_transform -- exact per-row top-k fused with the page-table transform.
 *
 * Defined by SGLang PR #26788 (Feature section; the raw-index commit note:
 * raw_out[i, j] is the pre-transform position chosen for slot j, or -1 for
 * padding, and out[j] equals the page transform of raw[j]) and LiteTopk PR
 * #32094 (Notes: an exact top-k *set* whose order within the row is
 * unspecified; sglang deviations: -1 pads invalid slots).
 *
 * Arguments (all pointers are device pointers on the current HIP device, read
 * or written only by kernels queued on `stream`):
 *   scores      (batch, width) fp32, row-major, contiguous.  Read only.
 *   seq_lens    (batch,) int32.  Row b uses positions [0, L_b) with
 *               L_b = clamp(seq_lens[b], 0, width).  Negative lengths are
 *               empty rows; lengths above width are read as width.
 *   page_table  (batch, pages_per_row) int32, row-major.  Only the entries of
 *               pages that hold a selected position are read.
 *   k           1 <= k <= TOPK_MAX_K; a runtime value.
 *   page_size   a power of two >= 1.
 *   out_idx     (batch, k) int32, written.  For slot j < n_b = min(k, L_b):
 *               page_table[b, p / page_size] * page_size + p % page_size for a
 *               selected position p; slots j >= n_b hold -1.
 *   out_raw     (batch, k) int32 or NULL.  When non-NULL, slot j holds the
 *               selected position p itself (same slot order as out_idx), and
 *               -1 in the same padding slots.  NULL costs nothing.
 *   stream      HIP stream the work is queued on (0 = the null stream).
 *   batch       number of rows, >= 0 (0 is a no-op).
 *   width       row stride of scores in elements, >= 0.
 *   pages_per_row  row stride of page_table in entries, >= 0.
 *
 * Result: slots [0, n_b) of each row hold n_b distinct positions in [0, L_b)
 * that are a top-n_b set of the row: every position whose score is strictly
 * greater than the smallest selected score is selected, and the remaining slots
 * take distinct positions whose score equals it.  Scores are ordered as IEEE
 * fp32 values with -0.0 below +0.0; -inf is an ordinary (selectable) value; NaN
 * is outside the contract.  Which of several equal scores fill the last slots,
 * and the order of the slots, are unspecified.
 *
 * Caller preconditions (not checked on the device, because checking would need
 * a host synchronisation): pages_per_row * page_size >= L_b for every row, and
 * every transformed index fits in int32.  A slot whose page lies beyond
 * pages_per_row gets -1 in out_idx (its raw position is still written).
 *
 * Ownership: the caller owns every buffer; the library keeps no pointer past
 * the call.  Rows split across workgroups, and batches with more rows than
 * the streaming kernel's grid, use an internal per-(device, stream) workspace
 * that the library allocates on first need, keeps in its initial state
 * between calls, and frees in topk_release_workspaces().  The first call
 * that needs a larger workspace allocates and clears it synchronously (so do
 * not make that first call under stream capture); the smaller one it replaces
 * stays allocated until topk_release_workspaces(), so graphs captured before
 * the growth stay valid.  The library also allocates, once per device, one
 * page of pinned host memory through which split launches report waits that
 * gave up (TOPK_ERROR_DEVICE_FAULT).
 *
 * Split rows rely on every workgroup of a row being resident at once: the
 * grid is sized to the device's resident capacity and launched normally (no
 * cooperative launch).  When a batch's rows cannot all be resident at once
 * they are cycled over the resident slots in one of two shapes (more
 * workgroups per row, or more rows at once), both held by one launch; the
 * device takes the one the row lengths favour (the first while the rows
 * longer than one of its workgroups fit two rounds of its slots).  The
 * dispatch override forces one.  If the workgroups of a row are not all
 * resident after all, a bounded wait gives up and the call's outputs are
 * invalid; this is reported as TOPK_ERROR_DEVICE_FAULT, never silently.
 *
 * Completion is asynchronous: outputs are valid once `stream` reaches the call.
 * Returns TOPK_SUCCESS, or an error status; on error nothing was queued.
 */
topk_status_t topk_transform(const float* scores, const int32_t* seq_lens, const int32_t* page_table,
                             int32_t k, int32_t page_size, int32_t* out_idx, int32_t* out_raw,
                             hipStream_t stream, int32_t batch, int64_t width, int64_t pages_per_row);

/*
 * Deterministic variant of topk_transform (same arguments, layouts, ownership
 * and errors).  LiteTopk PR #32094 (Notes) points out that the radix top-k
 * paths return an exact set in an unspecified order, with threshold ties
 * filled in atomic-arrival order, so they are not usable where a
 * deterministic result is required.  Here slots [0, n_b) of row b hold the
 * selected positions in the order of the plain definition: score descending
 * (the key order: IEEE order with -0 before +0), equal scores by position
 * ascending; where the threshold value is cut, the positions taken are the
 * lowest.  The output is therefore unique: the same for every kernel shape,
 * launch and device state.  out_idx[b, j] is the transform of out_raw[b, j];
 * slots [n_b, k) are -1.
 *
 * Cost: the row is selected as by topk_transform; then the selected
 * positions' scores are gathered (when ties at the threshold value are cut,
 * the row is read once more to take the lowest tied positions), and the n_b
 * chosen pairs are put in order: by one workgroup per row with a bitonic
 * network in LDS, or, for batches of fewer rows than CUs, by several
 * workgroups per row that each count, for their share of the pairs, the
 * larger pairs (topk_set_sorted_finish).
 * Besides the workspace, one 32-byte record and k raw positions per row are
 * kept per (device, stream) between the two launches; they are allocated on
 * first use (call once outside graph capture), grown on demand, and freed by
 * topk_release_workspaces.
 */
topk_status_t topk_transform_sorted(const float* scores, const int32_t* seq_lens, const int32_t* page_table,
                                    int32_t k, int32_t page_size, int32_t* out_idx, int32_t* out_raw,
                                    hipStream_t stream, int32_t batch, int64_t width, int64_t pages_per_row);

/*
 * topk_transform_noalloc -- topk_transform for callers that cannot allocate:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, layouts, result and errors as topk_transform;
 * it calls no allocating routine.  Its workspace is the library's static
 * device scratch (24 MiB per device, held from the library's first call on
 * the device until the process ends) instead of a per-(device, stream)
 * buffer.  The first call on a device that needs the scratch queues a zero
 * fill of it on `stream` before its own kernel.
 *
 * Limit: shapes whose split-row plan needs more than 152 row slots of
 * workspace return TOPK_ERROR_UNSUPPORTED with a message (no current plan
 * does: split rows are chosen only for fewer than half a row per CU).
 *
 * Every call on one device shares that device's scratch, and each call's
 * kernels leave it in its initial state; calls whose kernels overlap on one
 * device (queued on different streams without ordering between them) race
 * on it and give wrong results.  Split-row waits that give up are reported
 * as for topk_transform (TOPK_ERROR_DEVICE_FAULT at the next call of this
 * entry point, or from topk_check_faults); the next-call report needs the
 * pinned page topk_init() allocates.
 */
topk_status_t topk_transform_noalloc(const float* scores, const int32_t* seq_lens, const int32_t* page_table,
                                     int32_t k, int32_t page_size, int32_t* out_idx, int32_t* out_raw,
                                     hipStream_t stream, int32_t batch, int64_t width, int64_t pages_per_row);

/*
 * Sets up the current device for the library: device properties and kernel
 * residency, the static scratch's device address, and the pinned host page of
 * fault words.  Every entry point does this on its first call on a device
 * (topk_transform_noalloc without the page); calling it first, outside graph
 * capture, lets topk_transform_noalloc report faults at its next call too.
 * Returns TOPK_ERROR_UNSUPPORTED on a device that is not gfx950.
 */
topk_status_t topk_init(void);

/* Static text for a status code (never NULL). */
const char* topk_status_string(topk_status_t status);

/* Detail text of the most recent failing call on this host thread ("" if none). */
const char* topk_last_error(void);

/* Text naming the launch configuration of the most recent successful call on
 * this host thread (kernel variant, workgroups per row, elements per thread,
 * grid size).  For logs and benchmarks. */
const char* topk_last_launch(void);

/* Frees every internal workspace (after synchronising the device).  Safe to
 * call at any time no call is in flight. */
topk_status_t topk_release_workspaces(void);

/*
 * Testing and tuning override of the dispatcher, process-wide:
 *   elems_per_thread  0 = automatic, else one of 4, 8, 16, 32, 64: scores held
 *                     in registers per thread (a workgroup holds 1024 times
 *                     this many positions of a row);
 *   wgs_per_row       0 = automatic, else the number of workgroups that share
 *                     one row (raised to what the row width needs).  1 selects
 *                     the single-workgroup kernel.
 * Returns TOPK_ERROR_INVALID_VALUE for other values.
 */
topk_status_t topk_set_dispatch_override(int32_t elems_per_thread, int32_t wgs_per_row);

/*
 * Testing and tuning override of the streaming kernel's compiled shape,
 * process-wide: -1 = automatic (the dispatcher picks by batch and k), else
 *   0: 1024-thread workgroups, 16K-position sample, 8K-position chunks,
 *      6144 LDS candidates, 2 workgroups per CU (few rows, k up to 2048,
 *      rows with many tied keys);
 *   1: 256-thread workgroups, 8K-position sample, 4K-position chunks,
 *      1920 LDS candidates, 4 workgroups per CU (large batches, k <= 512);
 *   2: 1024-thread workgroups, 16K-position sample, three 16K-position
 *      chunks in flight, 6144 LDS candidates, 1 workgroup per CU (at most
 *      one row per two CUs, rows of 128K positions and more).
 * Every shape is exact for every input; the choice only moves time.
 * Returns TOPK_ERROR_INVALID_VALUE for other values.
 */
topk_status_t topk_set_stream_shape(int32_t shape);

/*
 * Testing and tuning override of the split streaming kernel, process-wide
 * (split streaming: G workgroups share a row, each streams a contiguous
 * segment behind its own sampled gate, and the last one to finish selects
 * from the merged lists):
 *   shape        -1 = automatic (the dispatcher decides), else a compiled
 *                shape forced for every call:
 *                  0: 1024-thread workgroups, two per CU, an 8K-position
 *                     sample, two 8K-position chunks in flight;
 *                  1: 1024-thread workgroups, one per CU, a 16K-position
 *                     sample, three 16K-position chunks in flight;
 *   wgs_per_row  G, 0 <= G <= 1024, when shape >= 0.  G = 0 selects the
 *                length-aware form: each row gets between 1 and 4
 *                workgroups, by its length against the batch's total
 *                positions spread over the CUs, worked out on the device.
 * A forced call whose batch * G workgroups do not fit resident at once (G
 * given), or with G above 4 or more than 256 rows, returns
 * TOPK_ERROR_UNSUPPORTED.  Every shape and G are exact for every
 * input; the choice only moves time.  Returns TOPK_ERROR_INVALID_VALUE for
 * other values.
 */
topk_status_t topk_set_split_stream(int32_t shape, int32_t wgs_per_row);

/*
 * Testing and tuning override of the sorted finish of topk_transform_sorted,
 * process-wide:
 *   -1  automatic: the rank finish for batches of fewer rows than CUs, else
 *       one workgroup per row;
 *    0  one workgroup per row, persistent over rows: the selected pairs are
 *       bitonic-sorted in LDS;
 *    1  the rank finish: G workgroups per row (about two per CU, at least 64
 *       pairs each) each compute the final slot of their share of the row's
 *       pairs by counting the larger pairs, bucketed by a data-fitted digit
 *       (a bucket crowded by tied keys is split again by a digit fitted to
 *       its own span; a row whose split stays crowded is sorted by its
 *       first workgroup as in mode 0).
 * Rows whose threshold bin was cut take the one-workgroup path in both
 * forms.  Both are exact for every input (the output is unique); the choice
 * only moves time.  Returns TOPK_ERROR_INVALID_VALUE for other values.
 */
topk_status_t topk_set_sorted_finish(int32_t mode);

/* Synchronises `stream`, then reports whether a split-row launch queued on
 * it (or, on this device, through topk_transform_noalloc) gave up a bounded
 * cross-workgroup wait since the last report: returns TOPK_ERROR_DEVICE_FAULT
 * once per such report (then TOPK_SUCCESS), with the detail in
 * topk_last_error().  The same report otherwise comes from the next call. */
topk_status_t topk_check_faults(hipStream_t stream);

/* Testing override, process-wide: the number of polls a split-row barrier
 * wait makes before it gives up (0 restores the default, on the order of a
 * second of waiting).  A tiny limit makes waits give up while every kernel
 * still runs to its end, which tests the TOPK_ERROR_DEVICE_FAULT report. */
topk_status_t topk_set_wait_limit(uint32_t polls);

/* Test knob: the number of 32-bit words of the static scratch that
 * topk_transform_noalloc may use (0, the default, = all of it; larger values
 * are the same as 0).  A plan whose workspace needs more is refused with
 * TOPK_ERROR_UNSUPPORTED, so a small value exercises that refusal with shapes
 * that fit the real scratch.  Process-wide; takes effect from the next call. */
topk_status_t topk_set_scratch_limit(uint64_t words);

/* ABI version of this header (bumped on any signature or export change). */
int32_t topk_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TOPK_TRANSFORM_H_ */
