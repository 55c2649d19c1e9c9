// Internal interface between the C-ABI layer (topk_api.cpp) and the gfx950
// kernels (topk_kernels.hip): launch parameters, workspace layout, launchers.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "topk_transform.h"

namespace topk {

// Per-host-thread status text shared by every entry point of the library.
void set_last_error(const char* msg);
void set_last_launch(const char* msg);

// The library's one lock: every entry point that touches the per-device or
// per-(device, stream) state holds it.
std::mutex& lib_mutex();

// A device buffer replaced by a larger one: kept allocated until
// topk_release_workspaces (a graph captured before the growth still names
// it).  Caller holds lib_mutex().
void retire_buffer(void* p);

// topk_transform for a caller that already holds lib_mutex().
topk_status_t transform_locked(const float* scores, const int32_t* seq_lens, const int32_t* page_table, int32_t k,
                               int32_t page_size, int32_t* out_idx, int32_t* out_raw, hipStream_t stream,
                               int32_t batch, int64_t width, int64_t pages_per_row);

constexpr int kThreads = 1024;          // threads per workgroup (16 wave64s)
constexpr int kWaves = kThreads / 64;
constexpr int kMaxK = 2048;
constexpr int kBinsWide = 4096;         // radix pass 0 digit: key bits 31..20
constexpr int kBinsNarrow = 1024;       // passes 1 and 2: key bits 19..10, 9..0
constexpr int kCandCap = 4096;          // threshold-bin candidates one workgroup finishes in LDS
constexpr int kSortSmallK = 512;        // sorted finish: k up to this takes the small workgroup shape
constexpr int kSortSmallThreads = 256;

// Elements per thread the kernels are instantiated for (register-resident keys).
constexpr int kNumEpt = 5;
constexpr int kEptValues[kNumEpt] = {4, 8, 16, 32, 64};

// ---------------------------------------------------------------------------
// Cross-workgroup workspace, in 32-bit words.  One region per (row slot,
// parity); rows handled by one slot alternate parity, so a region is never
// cleared while the slot's other workgroups already accumulate the next row.
// Every region is left zeroed by the workgroup that finishes its row.
// ---------------------------------------------------------------------------
// Header words, each group on its own 128-byte line; then the split streaming
// kernel's per-row counters.
constexpr size_t kSsMaxRows = 256;      // rows a split streaming launch may have
constexpr size_t kSsCtr = 128;          // per-row counters: 4 words per row
constexpr size_t kHdrWords = kSsCtr + 4 * kSsMaxRows;
constexpr size_t kHdrFault = 0;         // nonzero while a split launch in which a bounded wait gave up runs
constexpr size_t kHdrFaultCount = 1;    // split launches in which a wait gave up, ever (read by the host)
constexpr size_t kHdrRowTicket = 32;    // streaming kernel: rows handed out beyond the first grid's
constexpr size_t kHdrRowExit = 48;      // streaming kernel: workgroups out of rows
constexpr size_t kHdrLaunchExit = 64;   // split kernel: workgroups out of the current launch (+ 2^16 per give-up)
// Per-slot barrier block: an arrival counter per group of kBarGroup
// workgroups, a counter of completed groups, and the generation, each on its
// own 128-byte line (arrivals then contend per group, not per row, and the
// spinners' polls do not share a line with the atomics).
constexpr int kBarGroup = 8;
constexpr int kBarMaxGroups = 128;      // workgroups per row <= kBarGroup * kBarMaxGroups
constexpr size_t kBarLine = 32;         // words per 128-byte line
constexpr size_t kBarTop = kBarLine * kBarMaxGroups;
constexpr size_t kBarGen = kBarTop + kBarLine;
constexpr size_t kBarWords = kBarGen + kBarLine;
constexpr size_t kRegHist0 = 0;
constexpr size_t kRegHist1 = kRegHist0 + kBinsWide;
constexpr size_t kRegHist2 = kRegHist1 + kBinsNarrow;
constexpr size_t kRegCtr = kRegHist2 + kBinsNarrow;   // 64 words of counters
constexpr size_t kCtrSlots = 0;         // 64-bit: high word = slots taken by strictly-greater elements,
                                        // low word = tie slots / candidates appended
constexpr size_t kCtrExit = 32;         // workgroups done with the row
constexpr size_t kRegCandKey = kRegCtr + 64;
constexpr size_t kRegCandPos = kRegCandKey + kCandCap;
constexpr size_t kRegCandOut = kRegCandPos + kCandCap;   // each candidate's output value (page-table transform)
constexpr size_t kRegionWords = kRegCandOut + kCandCap;

inline size_t workspace_words(int64_t slots) {
  return kHdrWords + (size_t)slots * kBarWords + (size_t)slots * 2 * kRegionWords;
}
// Split-row slots a workspace of `words` words is laid out for.
inline int64_t workspace_slots(size_t words) {
  return words > kHdrWords ? (int64_t)((words - kHdrWords) / (kBarWords + 2 * kRegionWords)) : 0;
}

// Split streaming rows: four counters per row in the header (zero at rest;
// the row's finisher resets them), and an entry area per row after the
// header (kSsRowWords each).  The entry areas overlap the split-row layout,
// whose regions must be zero at rest; the finisher zeroes the entries it used.
constexpr size_t kSsExit = 0;           // 64-bit: workgroups done with the row, and each part's entry count
constexpr size_t kSsFloor = 2;          // the largest of the parts' gates (atomic max)
constexpr size_t kSsFlag = 3;           // nonzero: a part's list lost keys
constexpr int kSsMaxParts = 4;          // workgroups per row (parts) at most
constexpr int kSsExitBits = 4;          // exit word: bits [0, 4) count the parts out,
constexpr int kSsCountBits = 13;        // then 13 bits per part for its entry count
constexpr size_t kSsCap = 8192;         // entries an area holds (kSsCap / G per part)
constexpr size_t kSsKeys = 0;
constexpr size_t kSsPos = kSsKeys + kSsCap;
constexpr size_t kSsRowWords = kSsPos + kSsCap;
inline size_t split_stream_words(int64_t batch) { return kHdrWords + (size_t)batch * kSsRowWords; }

// Sorted mode: per-row selection record (prefix, shift, need, floor, cut,
// keys written).
constexpr size_t kMetaWords = 8;

struct KernelArgs {
  const float* scores;        // (batch, width)
  const int32_t* seq_lens;    // (batch,)
  const int32_t* page_table;  // (batch, pages_per_row)
  int32_t* out;               // (batch, k)
  int32_t* out_raw;           // (batch, k) or nullptr
  uint32_t* ws;               // workspace: split rows; streaming rows with batch > grid (row queue)
  int64_t width;
  int64_t pages_per_row;
  int32_t batch;
  int32_t k;
  int32_t log2_page;
  int32_t wgs_per_row;        // G: workgroups sharing one row
  int32_t slots;              // S: rows in flight; grid = S * G
  int32_t ws_slots;           // slots the workspace was laid out for (>= slots)
  int32_t vec;                // rows are 16-byte aligned: use dwordx4 loads
  uint32_t* meta;             // (batch, kMetaWords): how each row's selection ended, for the sorted finish; or nullptr
  const int32_t* sel;         // sorted finish: (batch, k) raw positions the selection launch wrote
  uint32_t* sel_key;          // sorted mode: (batch, k) order keys of those positions, written where a
                              // selection has them at hand (the record says so), else nullptr
  uint32_t spin_limit;        // split rows: polls of a barrier wait before it gives up
  uint32_t* fault_host;       // split rows: host-visible copy of the workspace's fault count, or nullptr
  int32_t spread;             // split streaming: 0 = wgs_per_row parts per row; else per-row parts from
                              // the lengths, at most wgs_per_row, the positions spread over this many shares
  // The cycled pair's kernel: it takes the E = 16 shape if at most
  // choice_rows rows are longer than choice_len positions, else the E = 64
  // shape.
  int32_t choice_rows;
  int32_t choice_len;
};

// Polls of a split-row barrier wait before it gives up (with s_sleep 1 between
// polls: on the order of a second).
constexpr uint32_t kDefaultSpinLimit = 1u << 21;

// ept_index selects kEptValues[ept_index]; coop selects the cross-workgroup
// kernel (cooperative launch, grid = slots * wgs_per_row).
hipError_t launch_rows(int ept_index, bool coop, const KernelArgs& args, hipStream_t stream);
hipError_t rows_occupancy(int ept_index, bool coop, int* blocks_per_cu);
// Cycled split rows in one launch that takes E = 64 (a.wgs_per_row, a.slots)
// or E = 16 (g16, slots16) from the row lengths (a.choice_rows,
// a.choice_len); grid = the larger of the two shapes' slots * wgs_per_row, all
// resident at once.
hipError_t launch_rows_pair(const KernelArgs& a, int32_t g16, int32_t slots16, hipStream_t stream);
hipError_t rows_pair_occupancy(int* blocks_per_cu);

// Streaming kernel, one workgroup per row, persistent over rows (grid =
// slots).  `variant` selects one of kNumStreamVariants compiled shapes
// (threads per workgroup, sample and chunk sizes, LDS candidate capacity).
constexpr int kNumStreamVariants = 3;
hipError_t launch_stream_rows(int variant, const KernelArgs& args, hipStream_t stream);
hipError_t stream_occupancy(int variant, int* blocks_per_cu);
int stream_variant_threads(int variant);

// Split streaming kernel: G workgroups per row (wgs_per_row), or per-row
// counts from the lengths (spread > 0); grid = batch * G.  `variant` selects
// a compiled shape.
constexpr int kNumSplitStreamVariants = 2;
hipError_t launch_split_stream(int variant, const KernelArgs& args, hipStream_t stream);
hipError_t split_stream_occupancy(int variant, int* blocks_per_cu);

// Sorted finish (deterministic mode): one workgroup per row, persistent over
// rows (grid = slots); reads the per-row records a selection launch left in
// `meta` and rewrites the row's outputs in canonical order.  The workgroup
// shape depends on k (kSortSmallK); sorted_occupancy reports the one for k.
hipError_t launch_sorted_rows(const KernelArgs& args, hipStream_t stream);
hipError_t sorted_occupancy(int k, int* blocks_per_cu);
// Rank finish (small batches): wgs_per_row workgroups per row, grid = batch *
// wgs_per_row, no synchronisation among them; each ranks its share of the
// row's selected pairs (rows whose bin was cut are finished by their first
// workgroup as in launch_sorted_rows).
hipError_t launch_sorted_rank(const KernelArgs& args, hipStream_t stream);

// The library's static device scratch: the workspace of the entry point that
// allocates nothing (topk_transform_noalloc).  One copy per device, 24 MiB,
// which holds the header and up to kScratchSlots (152) split-row slots.
constexpr size_t kScratchWords = (size_t)6 << 20;
constexpr int64_t kScratchSlots = (int64_t)((kScratchWords - kHdrWords) / (kBarWords + 2 * kRegionWords));
// Its address on the current device (hipGetSymbolAddress: the array's
// host-side name is not a device address).  Called once per device.
hipError_t scratch_address(uint32_t** ptr);
// Zero-fills `words` words at p with a kernel on `stream` (no memset node, so
// it may be captured in a graph).
hipError_t clear_words(uint32_t* p, size_t words, hipStream_t stream);

}  // namespace topk
