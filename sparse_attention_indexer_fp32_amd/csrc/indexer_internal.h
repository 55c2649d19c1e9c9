// Internal interface between the indexer C-ABI layer and its kernels.
#ifndef INDEXER_INTERNAL_H_
#define INDEXER_INTERNAL_H_

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace indexer {

// Arguments of both scoring kernels (dense logits and fused scan).
struct ScanArgs {
  const uint8_t* q;          // (num_q, 32, 128) fp8 E4M3 codes
  const float* weights;      // (num_q, 32)
  const uint8_t* kv;         // (num_kv, 128) fp8 E4M3 codes
  const float* kv_scale;     // (num_kv,)
  const int32_t* ks;         // (num_q,)
  const int32_t* ke;         // (num_q,)
  int64_t num_q;
  int64_t num_kv;
  int64_t window;            // key positions per window (multiple of 32)
  int32_t nwin;              // windows (grid.y)
  // dense logits
  float* logits;             // (num_q, logits_stride), row-relative columns
  int64_t logits_stride;
  // fused scan
  int32_t k;
  int32_t cap;               // candidate list capacity per (row, window)
  float* cand_score;         // (num_q, nwin, cap)
  int32_t* cand_pos;
  float* row_score;          // (num_q, row_cap): the row's candidates, packed
  int32_t* row_pos;
  int32_t* row_count;        // (num_q,)
  int64_t row_cap;
  // One window per row: the select reads each row's list in place (row_count
  // = the list's length, no final trim, no packed copy; row_score / row_pos
  // unused).
  int32_t inplace;
};

hipError_t launch_logits(const ScanArgs& a, int nwin, hipStream_t stream);
hipError_t launch_scan(const ScanArgs& a, int nwin, hipStream_t stream);
// Dense select of indexer_topk: len[r] = row r's clamped range length; out =
// rel (num_q x k row-relative positions, -1 padded) + each row's range start.
hipError_t launch_row_lengths(const ScanArgs& a, int32_t* len, hipStream_t stream);
hipError_t launch_absolute_positions(const ScanArgs& a, const int32_t* rel, int32_t* out, hipStream_t stream);
int rows_per_workgroup();

// The indexer's per-(device, stream) buffers: whether any are held, and
// freeing them (the caller has synchronised the device).
bool has_buffers();
void release_buffers();

}  // namespace indexer

#endif  // INDEXER_INTERNAL_H_
