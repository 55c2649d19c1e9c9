// C-ABI layer of the fused top-k + page-table transform: argument checks,
// device checks, the dispatcher that picks a kernel shape from the host-known
// (batch, width, k) and the device's resident-workgroup capacity, the
// per-(device, stream) buffers (the workspace the split-row kernel
// synchronises through, also the streaming kernel's row queue; the sorted
// mode's per-row records), and the report of split-row waits that gave up.
//
// Dispatch follows the pages' lesson that the path must depend on batch and
// length (SGLang PR #26788 commit notes: one block per row at large batch,
// several cooperating blocks per row for long rows at small batch), with the
// thresholds measured on MI355X (256 CUs): streaming from half a row per CU
// up, register-resident rows for a few short ones, split rows otherwise --
// cycled over the resident slots when they do not all fit at once and that
// is estimated faster than streaming them.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "indexer_internal.h"
#include "topk_internal.h"
#include "topk_transform.h"

namespace {

thread_local std::string t_last_error;
thread_local std::string t_last_launch;

// Words of a device's host-visible fault page: word 0 for the static scratch,
// then one per workspace.  A split launch whose bounded wait gave up stores its
// workspace's new fault count there.
constexpr int kFaultWords = 1024;

struct DeviceInfo {
  bool supported = false;
  int cus = 0;
  int occ[2][topk::kNumEpt] = {};   // [split][ept] resident workgroups per CU
  int stream_occ[topk::kNumStreamVariants] = {};   // streaming kernel shapes: resident workgroups per CU
  int sorted_occ_small = 0;         // sorted finish: resident workgroups per CU, k <= kSortSmallK
  int sorted_occ = 0;               //                                            larger k
  int ss_occ[topk::kNumSplitStreamVariants] = {};   // split streaming shapes: resident workgroups per CU
  int pair_occ = 0;                 // the cycled pair's kernel (E = 16 or 64): resident workgroups per CU
  uint32_t* fault_page = nullptr;   // pinned, device-mapped host memory (kFaultWords words), or null
  uint32_t* fault_page_dev = nullptr;   // its device address
  int fault_next = 1;               // next unassigned word of the page
  uint32_t* scratch = nullptr;      // device address of the static scratch
  bool scratch_zeroed = false;      // the scratch's zero fill has been queued
  uint32_t scratch_reported = 0;    // the scratch's fault count last reported
  std::string arch;
};

struct Workspace {
  uint32_t* ptr = nullptr;
  size_t words = 0;
  int fault_word = -1;              // this workspace's word of the device's fault page
  uint32_t reported = 0;            // its fault count last reported
};

// One lock for the whole library (the indexer entry points take it too, and
// hold it across their launches and the select that reads their buffers).
std::mutex& g_mu = topk::lib_mutex();
std::map<int, DeviceInfo> g_devices;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
std::map<std::pair<int, hipStream_t>, Workspace> g_meta;   // sorted mode: records + raw positions
// Buffers replaced by larger ones.  A graph captured before the growth still
// names them, so they stay allocated until topk_release_workspaces.
std::vector<void*> g_retired;
int g_override_ept = 0;
int g_override_wgs = 0;
int g_stream_variant = -1;   // -1: the default streaming shape
int g_ss_variant = -1;       // split streaming override: -1 automatic, else the shape forced
int g_sorted_finish = -1;    // sorted finish override: -1 automatic, 0 one workgroup per row, 1 rank finish
int g_ss_wgs = 0;            // ... with this many workgroups per row
uint32_t g_spin_limit = topk::kDefaultSpinLimit;
size_t g_scratch_limit = 0;  // words of the static scratch the no-allocation entry point may use; 0: all

topk_status_t fail(topk_status_t st, const std::string& msg) {
  t_last_error = msg;
  return st;
}

topk_status_t hip_fail(hipError_t e, const char* what) {
  return fail(TOPK_ERROR_LAUNCH, std::string(what) + ": " + hipGetErrorString(e));
}

// Caller holds g_mu.
topk_status_t device_info(int dev, DeviceInfo** out) {
  auto it = g_devices.find(dev);
  if (it != g_devices.end()) {
    *out = &it->second;
    return TOPK_SUCCESS;
  }
  hipDeviceProp_t prop;
  hipError_t e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  DeviceInfo info;
  info.arch = prop.gcnArchName;
  info.supported = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  info.cus = prop.multiProcessorCount;
  if (info.supported) {
    for (int c = 0; c < 2; ++c)
      for (int i = 0; i < topk::kNumEpt; ++i) {
        e = topk::rows_occupancy(i, c == 1, &info.occ[c][i]);
        if (e != hipSuccess) return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
      }
    for (int v = 0; v < topk::kNumStreamVariants; ++v) {
      e = topk::stream_occupancy(v, &info.stream_occ[v]);
      if (e != hipSuccess) return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
    }
    e = topk::sorted_occupancy(topk::kSortSmallK, &info.sorted_occ_small);
    if (e == hipSuccess) e = topk::sorted_occupancy(topk::kMaxK, &info.sorted_occ);
    if (e != hipSuccess) return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
    for (int v = 0; v < topk::kNumSplitStreamVariants; ++v) {
      e = topk::split_stream_occupancy(v, &info.ss_occ[v]);
      if (e != hipSuccess) return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
    }
    e = topk::rows_pair_occupancy(&info.pair_occ);
    if (e != hipSuccess) return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
    // set-up of the static scratch: its address on this (the current) device
    e = topk::scratch_address(&info.scratch);
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
  }
  *out = &g_devices.emplace(dev, info).first->second;
  return TOPK_SUCCESS;
}

// Caller holds g_mu.  The device's page of host-visible fault words.
topk_status_t ensure_fault_page(DeviceInfo& info) {
  if (info.fault_page != nullptr) return TOPK_SUCCESS;
  void* page = nullptr;
  hipError_t e = hipHostMalloc(&page, kFaultWords * sizeof(uint32_t), hipHostMallocMapped | hipHostMallocCoherent);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(TOPK_ERROR_OUT_OF_MEMORY, std::string("fault page hipHostMalloc: ") + hipGetErrorString(e));
  }
  std::memset(page, 0, kFaultWords * sizeof(uint32_t));
  void* page_dev = nullptr;
  e = hipHostGetDevicePointer(&page_dev, page, 0);
  if (e != hipSuccess) {
    (void)hipHostFree(page);
    return hip_fail(e, "hipHostGetDevicePointer");
  }
  info.fault_page = static_cast<uint32_t*>(page);
  info.fault_page_dev = static_cast<uint32_t*>(page_dev);
  return TOPK_SUCCESS;
}

// Caller holds g_mu.  `count` is a workspace's fault count (split launches on
// it whose bounded wait gave up); reports once each time it moves.  The device
// stores the count when such a launch ends, so a report can come one call
// late, or from topk_check_faults after a synchronisation.
topk_status_t take_fault(uint32_t count, uint32_t* reported) {
  if (count == 0u || count == *reported) return TOPK_SUCCESS;
  *reported = count;
  return fail(TOPK_ERROR_DEVICE_FAULT,
              "an earlier split-row launch on this stream gave up a cross-workgroup wait (its workgroups were not "
              "all resident at once); that launch's outputs are invalid and must be recomputed; this call queued "
              "nothing");
}

uint32_t page_word(const DeviceInfo& info, int word) {
  if (info.fault_page == nullptr || word < 0) return 0u;
  return __atomic_load_n(info.fault_page + word, __ATOMIC_ACQUIRE);
}

// Caller holds g_mu.
topk_status_t get_workspace(DeviceInfo& info, int dev, hipStream_t stream, size_t words, Workspace** out) {
  topk_status_t st = ensure_fault_page(info);
  if (st != TOPK_SUCCESS) return st;
  Workspace& w = g_ws[std::make_pair(dev, stream)];
  if (w.fault_word < 0) {
    w.fault_word = info.fault_next < kFaultWords ? info.fault_next++ : kFaultWords - 1;
  }
  *out = &w;
  if (w.ptr && w.words >= words) return TOPK_SUCCESS;
  const size_t bytes = words * sizeof(uint32_t);
  void* p = nullptr;
  if (std::getenv("TOPK_TEST_FAIL_ALLOC") == nullptr) {
    hipError_t e = hipMalloc(&p, bytes);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(TOPK_ERROR_OUT_OF_MEMORY, std::string("workspace hipMalloc: ") + hipGetErrorString(e));
    }
  } else {
    return fail(TOPK_ERROR_OUT_OF_MEMORY, "workspace allocation failure forced by TOPK_TEST_FAIL_ALLOC");
  }
  hipError_t e = hipMemsetAsync(p, 0, bytes, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  // a new buffer continues the stream's fault count, so reports stay one per fault
  if (e == hipSuccess && w.reported != 0u)
    e = hipMemcpy(static_cast<uint32_t*>(p) + topk::kHdrFaultCount, &w.reported, sizeof(uint32_t),
                  hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(p);
    return hip_fail(e, "workspace hipMemset");
  }
  if (w.ptr) g_retired.push_back(w.ptr);
  w.ptr = static_cast<uint32_t*>(p);
  w.words = words;
  return TOPK_SUCCESS;
}

// Caller holds g_mu.  Sorted mode's buffer: per-row selection records, then
// the selection launch's raw positions (batch x k) and the keys it writes
// beside them (batch x k).  Every row's record is written by the selection
// launch before the finish reads it, so the buffer needs no clearing.
topk_status_t get_meta(int dev, hipStream_t stream, int64_t words, uint32_t** ptr) {
  Workspace& w = g_meta[std::make_pair(dev, stream)];
  if (w.ptr && w.words >= (size_t)words) {
    *ptr = w.ptr;
    return TOPK_SUCCESS;
  }
  void* p = nullptr;
  hipError_t e = hipMalloc(&p, (size_t)words * sizeof(uint32_t));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(TOPK_ERROR_OUT_OF_MEMORY, std::string("selection record hipMalloc: ") + hipGetErrorString(e));
  }
  if (w.ptr) g_retired.push_back(w.ptr);
  w.ptr = static_cast<uint32_t*>(p);
  w.words = (size_t)words;
  *ptr = w.ptr;
  return TOPK_SUCCESS;
}

int ept_index(int ept) {
  for (int i = 0; i < topk::kNumEpt; ++i)
    if (topk::kEptValues[i] == ept) return i;
  return -1;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

enum class Kind { kResident, kSplit, kStream, kSplitStream };

// Preferred upper bound on workgroups sharing one split row.
constexpr int64_t kMaxSplitWgs = 128;

// Compiled streaming shapes (TOPK_STREAM_VARIANTS): 0 = 1024-thread
// workgroups with 6144 LDS candidates, two per CU; 1 = 256-thread workgroups
// with 1920, four per CU; 2 = 1024-thread workgroups, one per CU, with three
// 16K-position chunks (192 KB) in flight instead of two 8K ones.
constexpr int kStreamWide = 0;
constexpr int kStreamNarrow = 1;
constexpr int kStreamDeep = 2;

struct Plan {
  Kind kind = Kind::kStream;
  int stream_variant = kStreamWide;
  int ss_variant = 0;
  bool ss_spread = false;   // split streaming: per-row parts from the lengths (G is their maximum)
  int ept_idx = 0;
  int64_t G = 1;
  int64_t slots = 1;
  // Cycled split rows: a second shape (smaller E, more workgroups per row)
  // launched before this one; the device picks one of the two from the row
  // lengths (alt_ept_idx < 0: none)
  int alt_ept_idx = -1;
  int64_t alt_G = 0;
  int64_t alt_slots = 0;
};

const char* kind_name(Kind k) {
  switch (k) {
    case Kind::kResident: return "row-per-wg-resident";
    case Kind::kSplit: return "split-row";
    case Kind::kStream: return "row-per-wg-stream";
    case Kind::kSplitStream: return "split-row-stream";
  }
  return "?";
}

// Kernel shape for (batch, width, k) on this device.
//  * stream:   one workgroup per row, rows streamed from HBM past a gate set
//              from a sample; persistent over rows (a queue hands out the rows
//              beyond the grid).  Used from half a row per CU up (measured on
//              MI355X: at 128 rows of 128K it beats the split kernel by a
//              quarter).  The 256-thread shape (four
//              workgroups per CU) when the batch fills its slots and k <= 512
//              (its 1920-entry list holds the ~2k keys such rows pass), else
//              the 1024-thread shape.
//  * split:    G workgroups per row holding the row in registers, merged
//              through global atomics and a per-row barrier; for fewer, long
//              rows.  Picks the smallest E whose grid still fits resident;
//              when none does, E = 64 with the rows cycled over the resident
//              slots, if that is estimated faster than streaming them.
//  * resident: one workgroup per row holding the row in registers; for
//              fewer than half a row per CU of width <= 16K.
topk_status_t plan_launch(const DeviceInfo& dev, int32_t batch, int64_t width, int32_t k, Plan* plan) {
  const int64_t B = batch;
  const int64_t Wc = width > 0 ? width : 1;
  // The deep shape for at most one row per two CUs of width >= 128K: each
  // row's workgroup streams alone, limited by what it keeps in flight
  // (measured on MI355X: 128 x 128K, k 512: 27.9 against 29.4 us; 128 x 128K
  // ties, k 1024: 32.5 against 33.9 us; but 256 x 128K: 38.1 against 33.3 us
  // and 128 x 64K: 24.1 against 23.6 us).
  if (g_stream_variant >= 0)
    plan->stream_variant = g_stream_variant;
  else if (k <= 512 && B >= (int64_t)dev.stream_occ[kStreamNarrow] * dev.cus)
    plan->stream_variant = kStreamNarrow;
  else if (2 * B <= (int64_t)dev.cus && Wc >= 131072)
    plan->stream_variant = kStreamDeep;
  else
    plan->stream_variant = kStreamWide;
  const int64_t stream_slots = (int64_t)dev.stream_occ[plan->stream_variant] * dev.cus;
  auto split_ept_for = [&](int64_t wgs) {   // smallest E whose G for this width is <= wgs
    int idx = 0;
    while (idx < topk::kNumEpt - 1 && (int64_t)topk::kThreads * topk::kEptValues[idx] * wgs < Wc) ++idx;
    return idx;
  };

  // split streaming: G workgroups per row, all resident at once; or, with
  // `spread`, up to G per row from the rows' lengths (no residency needed:
  // no workgroup of this kernel waits for another)
  auto split_stream = [&](int variant, int64_t G, bool spread = false) -> topk_status_t {
    const int64_t cap = (int64_t)dev.ss_occ[variant] * dev.cus;
    if (G < 1 || G > topk::kSsMaxParts || (!spread && B * G > cap) || B > (int64_t)topk::kSsMaxRows)
      return fail(TOPK_ERROR_UNSUPPORTED,
                  "split streaming takes at most 4 workgroups per row and 256 rows, all resident at once");
    plan->kind = Kind::kSplitStream;
    plan->ss_variant = variant;
    plan->ss_spread = spread;
    plan->G = G;
    plan->slots = B;
    return TOPK_SUCCESS;
  };
  if (g_ss_variant >= 0)
    return g_ss_wgs > 0 ? split_stream(g_ss_variant, g_ss_wgs) : split_stream(g_ss_variant, topk::kSsMaxParts, true);
  // Split streaming rows, where measured to win.  G = CUs / B (2 to 4):
  // about one workgroup per CU, each streaming a segment of the row.  Only
  // where a row's merged candidates stay well inside the finisher's list:
  // the sample (8K positions) sets each segment's gate at the rank
  // m = mu + 7 sqrt(mu) + 6 of its n * S / L expected top keys, so a row
  // passes about m * L / S keys; rows whose lists would crowd the list fall
  // back to re-reading the row, which costs several times more (1M rows at
  // k 2048: 279 against 76 us).
  const int64_t ss_G = std::min<int64_t>(topk::kSsMaxParts, std::max<int64_t>(2, dev.cus / std::max<int64_t>(B, 1)));
  auto split_stream_fits = [&](double bound = 4500.0) {
    const double S = 8192.0, L = (double)Wc, n = (double)std::min<int64_t>(k, Wc);
    const double mu = n * std::min(S, L) / L;
    const double passed = (mu + 7.0 * std::sqrt(mu) + 6.0) * L / S;
    return g_stream_variant < 0 && B <= (int64_t)topk::kSsMaxRows && passed <= bound &&
           (int64_t)dev.ss_occ[0] * dev.cus >= ss_G * B;
  };
  if (g_override_ept || g_override_wgs) {
    if (g_override_wgs == 1 && g_override_ept == 0) {
      plan->kind = Kind::kStream;
    } else {
      const int idx = g_override_ept ? ept_index(g_override_ept) : split_ept_for(g_override_wgs);
      const int64_t C = (int64_t)topk::kThreads * topk::kEptValues[idx];
      int64_t G = ceil_div(Wc, C);
      if (g_override_wgs > G) G = g_override_wgs;
      plan->ept_idx = idx;
      plan->G = G;
      plan->kind = G > 1 ? Kind::kSplit : Kind::kResident;
    }
  } else if (2 * B >= dev.cus || B >= stream_slots) {
    // One row per two CUs, rows of 128K and more: two workgroups per row put
    // every CU to work (measured on MI355X: 128 x 128K, k 512: 24.4 against
    // 30.1 us; the tie-heavy 128 x 128K, k 1024: 27.4 against 34.1 us; 96 x
    // 128K, k 1024: 24.9 us).
    if (plan->stream_variant == kStreamDeep && split_stream_fits()) return split_stream(0, ss_G);
    plan->kind = Kind::kStream;
  } else if (B >= 32 && Wc >= 32768 && Wc <= 262144 && split_stream_fits()) {
    // Mid batches of rows up to 256K: G workgroups per row stream a segment
    // each, with no barrier, where split rows would hold the row in
    // registers behind one (measured on MI355X at k 2048: 64 ragged rows of
    // 4K-64K 18.9 against 23.1 us; 64 x 256K 28.6 against 43.9 us; 48 x 96K
    // 20.0 us; 32 x 128K 21.1 against 23.2 us; at k 512, 64 x 64K 15.4
    // against 21.1 us and 32 x 256K 22.3 us).  Fewer rows stay split: 16 x
    // 256K 22.8 us split against 26.0 us.
    return split_stream(0, ss_G);
  } else if (B >= 32 && Wc > 262144 && split_stream_fits(6000.0)) {
    // Mid batches of wider rows: the width says little about the lengths, so
    // each row gets 1 to 4 workgroups by its own length, worked out on the
    // device (measured on MI355X against split rows: 64 x 512K, k 512: 35.2
    // against 67.6 us; 32 x 1M, k 512: 51.2 against 66.7 us; 64 x 512K, k
    // 2048: 40.6 against 78.8 us; 48 rows of U[64K, 1M], k 1024: 53.2 against
    // 94.6 us; 64 rows of U[32K, 512K], k 1024: 35.4 against 70.8 us).
    return split_stream(0, topk::kSsMaxParts, true);
  } else if (Wc <= (int64_t)topk::kThreads * 16) {
    // few short rows: one workgroup each, the row in registers (1 x 16K, k 512:
    // 10.2 us against 12.6 us streamed)
    int idx = 0;
    while (idx < topk::kNumEpt - 1 && (int64_t)topk::kThreads * topk::kEptValues[idx] < Wc) ++idx;
    plan->ept_idx = idx;
    plan->G = 1;
    plan->kind = Kind::kResident;
  } else {
    // Smallest E whose grid fits resident with at most kMaxSplitWgs
    // workgroups per row: each extra workgroup adds histogram pushes and
    // barrier arrivals (measured on a 1M row: 256 workgroups 22 us, 128 19 us).
    int chosen = -1;
    for (int pass = 0; pass < 2 && chosen < 0; ++pass)
      for (int i = 0; i < topk::kNumEpt; ++i) {
        const int64_t G = ceil_div(Wc, (int64_t)topk::kThreads * topk::kEptValues[i]);
        const int64_t cap = (int64_t)dev.occ[1][i] * dev.cus;
        if (B * G <= cap && (pass == 1 || G <= kMaxSplitWgs)) {
          chosen = i;
          break;
        }
      }
    if (chosen < 0) {
      // No E holds every row resident at once.  The rows can still run as
      // split rows cycled over cap / G slots (E = 64: the fewest workgroups
      // per row), or stream one row per workgroup.  Measured on MI355X at
      // k 2048: a split iteration of full 64K-position workgroups takes
      // ~36 us; a streamed row moves ~27 GB/s on its one workgroup, plus
      // ~10 us.  The cheaper estimate wins: 32 x 1M rows 73 us split against
      // 153 us streamed, 4 x 1M + 28 x 16K 53 against 136, 16 x 2M 72
      // against 277; but 100 x 256K 73 against 54, and 120 x 512K (k 512)
      // 120 against 81, stay streamed.
      const int i = topk::kNumEpt - 1;
      const int64_t G = ceil_div(Wc, (int64_t)topk::kThreads * topk::kEptValues[i]);
      const int64_t cap = (int64_t)dev.occ[1][i] * dev.cus;
      const int64_t slots = cap / G;
      if (G > 1 && slots >= 1 && G <= (int64_t)topk::kBarGroup * topk::kBarMaxGroups) {
        const double t_split = 36.0 * (double)ceil_div(B, slots);
        const double t_stream = 4.0 * (double)Wc / 27000.0 + 10.0;
        if (t_split < t_stream) chosen = i;
      }
      // The estimate above assumes every row is long.  When few are (a
      // decode batch of a few long requests among short ones), E = 16 with
      // four times the workgroups per row finishes them in one round, and the
      // short rows run on one workgroup each meanwhile (measured on MI355X:
      // 4 x 1M + 28 x 16K, k 2048: 30.1-30.5 us at E 16 against 45.9-46.5 us
      // at E 64; 32 x 1M: 147 against 72.8 us).  Only the device knows the
      // lengths, so one launch holds both shapes, and its workgroups count
      // the rows that need more than one E = 16 workgroup: E = 16 runs if
      // they fit two rounds of its slots, else E = 64 (32 x 1M batches with
      // n such rows, the rest at most 16K, E 16 against E 64: n = 4 29.6
      // against 47.3 us; 6: 44.1 against 48.8; 8: 44.9 against 49.7; 12:
      // 61.0 against 54.4).  Both shapes' grids must fit the pair kernel's
      // residency.
      const int a16 = 2;   // kEptValues[2] = 16
      const int64_t G16 = ceil_div(Wc, (int64_t)topk::kThreads * topk::kEptValues[a16]);
      const int64_t slots16 = (int64_t)dev.pair_occ * dev.cus / G16;
      if (chosen == i && dev.pair_occ >= dev.occ[1][i] && slots16 >= 1 && slots16 < B &&
          G16 <= (int64_t)topk::kBarGroup * topk::kBarMaxGroups) {
        plan->alt_ept_idx = a16;
        plan->alt_G = G16;
        plan->alt_slots = slots16;
      }
    }
    if (chosen < 0) {
      // too many rows to hold resident: stream them, G workgroups per row
      // where that fits (100 x 256K at k 2048: 38.6 against 46.9 us streamed
      // one per workgroup; 120 x 512K at k 512: 54.5 against 65.1 us)
      if (plan->stream_variant == kStreamDeep && split_stream_fits()) return split_stream(0, ss_G);
      plan->kind = Kind::kStream;
    } else {
      plan->ept_idx = chosen;
      plan->G = ceil_div(Wc, (int64_t)topk::kThreads * topk::kEptValues[chosen]);
      plan->kind = plan->G > 1 ? Kind::kSplit : Kind::kStream;
    }
  }
  switch (plan->kind) {
    case Kind::kStream:
      plan->G = 1;
      plan->slots = B < stream_slots ? B : stream_slots;
      if (plan->slots < 1) plan->slots = 1;
      break;
    case Kind::kResident:
      plan->slots = B;
      break;
    case Kind::kSplitStream:
      break;
    case Kind::kSplit: {
      const int64_t cap = (int64_t)dev.occ[1][plan->ept_idx] * dev.cus;
      if (plan->G > cap || plan->G > (int64_t)topk::kBarGroup * topk::kBarMaxGroups)
        return fail(TOPK_ERROR_UNSUPPORTED, "row width needs more cooperating workgroups than fit resident");
      int64_t slots = cap / plan->G;
      if (slots > B) slots = B;
      plan->slots = slots;
      break;
    }
  }
  return TOPK_SUCCESS;
}

// Caller holds g_mu.  With `noalloc` (never with `sorted`) the workspace is
// the device's static scratch and nothing is allocated.
topk_status_t run_transform_locked(const float* scores, const int32_t* seq_lens, const int32_t* page_table,
                                   int32_t k, int32_t page_size, int32_t* out_idx, int32_t* out_raw,
                                   hipStream_t stream, int32_t batch, int64_t width, int64_t pages_per_row,
                                   bool sorted, bool noalloc = false) {
  t_last_error.clear();
  if (k < 1 || k > TOPK_MAX_K) return fail(TOPK_ERROR_INVALID_VALUE, "k must be in [1, 2048]");
  if (page_size < 1 || (page_size & (page_size - 1)) != 0)
    return fail(TOPK_ERROR_INVALID_VALUE, "page_size must be a power of two >= 1");
  if (batch < 0 || width < 0 || pages_per_row < 0)
    return fail(TOPK_ERROR_INVALID_VALUE, "batch, width and pages_per_row must be >= 0");
  if (width > (int64_t)INT32_MAX) return fail(TOPK_ERROR_INVALID_VALUE, "width must fit in int32");
  if (batch == 0) {
    t_last_launch = "noop batch=0";
    return TOPK_SUCCESS;
  }
  if (!seq_lens || !out_idx) return fail(TOPK_ERROR_INVALID_VALUE, "seq_lens and out_idx must be non-null");
  if (!scores && width > 0) return fail(TOPK_ERROR_INVALID_VALUE, "scores must be non-null when width > 0");
  if (!page_table && pages_per_row > 0)
    return fail(TOPK_ERROR_INVALID_VALUE, "page_table must be non-null when pages_per_row > 0");

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");

  DeviceInfo* info = nullptr;
  topk_status_t st = device_info(dev, &info);
  if (st != TOPK_SUCCESS) return st;
  if (!info->supported) return fail(TOPK_ERROR_UNSUPPORTED, "device " + info->arch + " is not gfx950");
  if (noalloc) {
    st = take_fault(page_word(*info, 0), &info->scratch_reported);
    if (st != TOPK_SUCCESS) return st;
  } else {
    auto wit = g_ws.find(std::make_pair(dev, stream));
    if (wit != g_ws.end()) {
      st = take_fault(page_word(*info, wit->second.fault_word), &wit->second.reported);
      if (st != TOPK_SUCCESS) return st;
    }
  }

  Plan plan;
  st = plan_launch(*info, batch, width, k, &plan);
  if (st != TOPK_SUCCESS) return st;

  topk::KernelArgs a{};
  a.scores = scores;
  a.seq_lens = seq_lens;
  a.page_table = page_table;
  a.out = out_idx;
  a.out_raw = out_raw;
  a.ws = nullptr;
  a.ws_slots = 0;
  a.width = width;
  a.pages_per_row = pages_per_row;
  a.batch = batch;
  a.k = k;
  int lg = 0;
  while ((1 << lg) < page_size) ++lg;
  a.log2_page = lg;
  a.wgs_per_row = (int32_t)plan.G;
  a.slots = (int32_t)plan.slots;
  a.vec = (width % 4 == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0) ? 1 : 0;
  a.meta = nullptr;
  a.sel = nullptr;
  a.sel_key = nullptr;
  a.spin_limit = g_spin_limit;
  a.fault_host = nullptr;
  a.spread = plan.kind == Kind::kSplitStream && plan.ss_spread ? info->cus : 0;
  if (sorted) {
    // the selection launch writes its raw positions to a scratch area after
    // the records, never to the caller's out_raw: the rank finish's
    // workgroups read a row's positions while others of the row write its
    // output
    const int64_t rec = (int64_t)batch * (int64_t)topk::kMetaWords;
    st = get_meta(dev, stream, rec + 2 * (int64_t)batch * k, &a.meta);
    if (st != TOPK_SUCCESS) return st;
    a.out_raw = reinterpret_cast<int32_t*>(a.meta + rec);
    a.sel = a.out_raw;
    a.sel_key = a.meta + rec + (int64_t)batch * k;
  }
  if (plan.kind == Kind::kSplit || plan.kind == Kind::kSplitStream ||
      (plan.kind == Kind::kStream && batch > plan.slots)) {
    // split rows synchronise through per-slot regions, split streaming rows
    // through per-row areas; streamed rows beyond the grid are handed out
    // through a counter in the header
    const size_t words = plan.kind == Kind::kSplit         ? topk::workspace_words(std::max(plan.slots, plan.alt_slots))
                         : plan.kind == Kind::kSplitStream ? topk::split_stream_words(batch)
                                                           : topk::kHdrWords;
    if (noalloc) {
      const size_t limit =
          g_scratch_limit != 0 && g_scratch_limit < topk::kScratchWords ? g_scratch_limit : topk::kScratchWords;
      if (words > limit) {
        char msg[200];
        std::snprintf(msg, sizeof(msg),
                      "this shape needs %zu words of workspace; the static scratch of the no-allocation entry "
                      "point holds %zu (%zu MiB)",
                      words, limit, (topk::kScratchWords * 4) >> 20);
        return fail(TOPK_ERROR_UNSUPPORTED, msg);
      }
      if (!info->scratch_zeroed) {
        e = topk::clear_words(info->scratch, topk::kScratchWords, stream);
        if (e != hipSuccess) return hip_fail(e, "scratch zero fill");
        info->scratch_zeroed = true;
      }
      a.ws = info->scratch;
      a.ws_slots = (int32_t)topk::kScratchSlots;
      a.fault_host = info->fault_page_dev;   // word 0, or none before a page exists
    } else {
      Workspace* w = nullptr;
      st = get_workspace(*info, dev, stream, words, &w);
      if (st != TOPK_SUCCESS) return st;
      a.ws = w->ptr;
      a.ws_slots = (int32_t)topk::workspace_slots(w->words);
      a.fault_host = info->fault_page_dev + w->fault_word;
    }
  }
  if (plan.kind == Kind::kStream)
    e = topk::launch_stream_rows(plan.stream_variant, a, stream);
  else if (plan.kind == Kind::kSplitStream)
    e = topk::launch_split_stream(plan.ss_variant, a, stream);
  else if (plan.alt_ept_idx >= 0) {
    // the pair of cycled shapes (Plan): E = 64 with this plan's workgroups
    // per row and slots, E = 16 with the alternative's; one launch, the
    // device takes one of them
    a.choice_rows = (int32_t)(2 * plan.alt_slots);
    a.choice_len = topk::kThreads * topk::kEptValues[plan.alt_ept_idx];
    e = topk::launch_rows_pair(a, (int32_t)plan.alt_G, (int32_t)plan.alt_slots, stream);
  } else
    e = topk::launch_rows(plan.ept_idx, plan.kind == Kind::kSplit, a, stream);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  int64_t sorted_slots = 0, sorted_g = 0;
  if (sorted) {
    // the finish reads every row's record once the selection launch is done (stream order)
    topk::KernelArgs f = a;
    f.out_raw = out_raw;   // the caller's (or none); f.sel holds the selection launch's positions
    // the rank finish, G workgroups per row (at least 64 pairs each; about
    // two 256-thread workgroups per CU for k <= 512, one 1024-thread
    // workgroup per CU above, the most MI355X holds at once of that shape),
    // unless the one-workgroup-per-row finish is forced
    const bool rank = g_sorted_finish != 0;
    if (rank) {
      int64_t G = (k <= topk::kSortSmallK ? 2 : 1) * (int64_t)info->cus / batch;
      if (G > k / 64) G = k / 64;
      if (G < 1) G = 1;
      sorted_g = G;
      f.slots = batch;
      f.wgs_per_row = (int32_t)G;
      e = topk::launch_sorted_rank(f, stream);
    } else {
      sorted_slots = (int64_t)(k <= topk::kSortSmallK ? info->sorted_occ_small : info->sorted_occ) * info->cus;
      if (sorted_slots > batch) sorted_slots = batch;
      if (sorted_slots < 1) sorted_slots = 1;
      f.slots = (int32_t)sorted_slots;
      f.wgs_per_row = 1;
      e = topk::launch_sorted_rows(f, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "sorted finish launch");
  }
  char sorted_note[64] = "";
  if (sorted)
    std::snprintf(sorted_note, sizeof(sorted_note), sorted_g > 0 ? " + sorted-finish rank G=%lld" : " + sorted-finish rows",
                  (long long)sorted_g);
  char pair_note[160] = "";
  if (plan.alt_ept_idx >= 0)
    std::snprintf(pair_note, sizeof(pair_note),
                  " | ept=%d wgs_per_row=%lld slots=%lld when at most %lld rows exceed %d positions (device "
                  "choice in one launch, grid=%lld)",
                  topk::kEptValues[plan.alt_ept_idx], (long long)plan.alt_G, (long long)plan.alt_slots,
                  (long long)(2 * plan.alt_slots), topk::kThreads * topk::kEptValues[plan.alt_ept_idx],
                  (long long)std::max(plan.alt_slots * plan.alt_G, plan.slots * plan.G));
  char buf[400];
  std::snprintf(buf, sizeof(buf), "%s%s ept=%d wgs_per_row=%lld slots=%lld grid=%lld block=%d vec=%d%s%s%s",
                kind_name(plan.kind), plan.ss_spread ? " length-aware" : "",
                plan.kind == Kind::kStream || plan.kind == Kind::kSplitStream ? 0 : topk::kEptValues[plan.ept_idx],
                (long long)plan.G, (long long)plan.slots, (long long)(plan.slots * plan.G),
                plan.kind == Kind::kStream ? topk::stream_variant_threads(plan.stream_variant) : topk::kThreads, a.vec,
                pair_note, sorted_note, noalloc ? " (static scratch)" : "");
  t_last_launch = buf;
  return TOPK_SUCCESS;
}

topk_status_t run_transform(const float* scores, const int32_t* seq_lens, const int32_t* page_table, int32_t k,
                            int32_t page_size, int32_t* out_idx, int32_t* out_raw, hipStream_t stream, int32_t batch,
                            int64_t width, int64_t pages_per_row, bool sorted) {
  std::lock_guard<std::mutex> lock(g_mu);
  return run_transform_locked(scores, seq_lens, page_table, k, page_size, out_idx, out_raw, stream, batch, width,
                              pages_per_row, sorted);
}

}  // namespace

namespace topk {
void set_last_error(const char* msg) { t_last_error = msg; }
void set_last_launch(const char* msg) { t_last_launch = msg; }
void retire_buffer(void* p) {
  if (p) g_retired.push_back(p);
}
std::mutex& lib_mutex() {
  static std::mutex m;
  return m;
}
topk_status_t transform_locked(const float* scores, const int32_t* seq_lens, const int32_t* page_table, int32_t k,
                               int32_t page_size, int32_t* out_idx, int32_t* out_raw, hipStream_t stream,
                               int32_t batch, int64_t width, int64_t pages_per_row) {
  return run_transform_locked(scores, seq_lens, page_table, k, page_size, out_idx, out_raw, stream, batch, width,
                              pages_per_row, false);
}
}  // namespace topk

extern "C" {

topk_status_t topk_transform(const float* scores, const int32_t* seq_lens, const int32_t* page_table, int32_t k,
                             int32_t page_size, int32_t* out_idx, int32_t* out_raw, hipStream_t stream,
                             int32_t batch, int64_t width, int64_t pages_per_row) {
  return run_transform(scores, seq_lens, page_table, k, page_size, out_idx, out_raw, stream, batch, width,
                       pages_per_row, false);
}

topk_status_t topk_transform_sorted(const float* scores, const int32_t* seq_lens, const int32_t* page_table,
                                    int32_t k, int32_t page_size, int32_t* out_idx, int32_t* out_raw,
                                    hipStream_t stream, int32_t batch, int64_t width, int64_t pages_per_row) {
  return run_transform(scores, seq_lens, page_table, k, page_size, out_idx, out_raw, stream, batch, width,
                       pages_per_row, true);
}

topk_status_t topk_transform_noalloc(const float* scores, const int32_t* seq_lens, const int32_t* page_table,
                                     int32_t k, int32_t page_size, int32_t* out_idx, int32_t* out_raw,
                                     hipStream_t stream, int32_t batch, int64_t width, int64_t pages_per_row) {
  std::lock_guard<std::mutex> lock(g_mu);
  return run_transform_locked(scores, seq_lens, page_table, k, page_size, out_idx, out_raw, stream, batch, width,
                              pages_per_row, false, true);
}

topk_status_t topk_init(void) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_mu);
  t_last_error.clear();
  DeviceInfo* info = nullptr;
  topk_status_t st = device_info(dev, &info);
  if (st != TOPK_SUCCESS) return st;
  if (!info->supported) return fail(TOPK_ERROR_UNSUPPORTED, "device " + info->arch + " is not gfx950");
  return ensure_fault_page(*info);
}

const char* topk_status_string(topk_status_t status) {
  switch (status) {
    case TOPK_SUCCESS: return "TOPK_SUCCESS";
    case TOPK_ERROR_INVALID_VALUE: return "TOPK_ERROR_INVALID_VALUE";
    case TOPK_ERROR_UNSUPPORTED: return "TOPK_ERROR_UNSUPPORTED";
    case TOPK_ERROR_OUT_OF_MEMORY: return "TOPK_ERROR_OUT_OF_MEMORY";
    case TOPK_ERROR_LAUNCH: return "TOPK_ERROR_LAUNCH";
    case TOPK_ERROR_DEVICE_FAULT: return "TOPK_ERROR_DEVICE_FAULT";
  }
  return "TOPK_UNKNOWN_STATUS";
}

const char* topk_last_error(void) { return t_last_error.c_str(); }

const char* topk_last_launch(void) { return t_last_launch.c_str(); }

topk_status_t topk_release_workspaces(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ws.empty() && g_meta.empty() && g_retired.empty() && !indexer::has_buffers()) return TOPK_SUCCESS;
  hipError_t e = hipDeviceSynchronize();
  indexer::release_buffers();
  // A released workspace's pending fault report goes with it: a stream's next
  // workspace gets a fresh fault word.
  for (auto& kv : g_ws)
    if (kv.second.ptr) (void)hipFree(kv.second.ptr);
  g_ws.clear();
  for (auto& kv : g_meta)
    if (kv.second.ptr) (void)hipFree(kv.second.ptr);
  g_meta.clear();
  for (void* p : g_retired) (void)hipFree(p);
  g_retired.clear();
  if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
  return TOPK_SUCCESS;
}

topk_status_t topk_set_dispatch_override(int32_t elems_per_thread, int32_t wgs_per_row) {
  if (elems_per_thread != 0 && ept_index(elems_per_thread) < 0)
    return fail(TOPK_ERROR_INVALID_VALUE, "elems_per_thread must be 0, 4, 8, 16, 32 or 64");
  if (wgs_per_row < 0 || wgs_per_row > 65536) return fail(TOPK_ERROR_INVALID_VALUE, "wgs_per_row out of range");
  std::lock_guard<std::mutex> lock(g_mu);
  g_override_ept = elems_per_thread;
  g_override_wgs = wgs_per_row;
  return TOPK_SUCCESS;
}

topk_status_t topk_set_split_stream(int32_t shape, int32_t wgs_per_row) {
  if (shape < -1 || shape >= topk::kNumSplitStreamVariants)
    return fail(TOPK_ERROR_INVALID_VALUE, "shape must be -1 (automatic) or a compiled split streaming shape index");
  if (shape >= 0 && (wgs_per_row < 0 || wgs_per_row > 1024))
    return fail(TOPK_ERROR_INVALID_VALUE, "wgs_per_row must be in [0, 1024]");
  std::lock_guard<std::mutex> lock(g_mu);
  g_ss_variant = shape;
  g_ss_wgs = shape >= 0 ? wgs_per_row : 0;
  return TOPK_SUCCESS;
}

topk_status_t topk_set_stream_shape(int32_t shape) {
  if (shape < -1 || shape >= topk::kNumStreamVariants)
    return fail(TOPK_ERROR_INVALID_VALUE, "shape must be -1 (default) or a compiled streaming shape index");
  std::lock_guard<std::mutex> lock(g_mu);
  g_stream_variant = shape;
  return TOPK_SUCCESS;
}

topk_status_t topk_set_sorted_finish(int32_t mode) {
  if (mode < -1 || mode > 1) return fail(TOPK_ERROR_INVALID_VALUE, "mode must be -1 (automatic), 0 or 1");
  std::lock_guard<std::mutex> lock(g_mu);
  g_sorted_finish = mode;
  return TOPK_SUCCESS;
}

topk_status_t topk_check_faults(hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_mu);
  t_last_error.clear();
  auto dit = g_devices.find(dev);
  if (dit == g_devices.end()) return TOPK_SUCCESS;
  DeviceInfo& info = dit->second;
  auto it = g_ws.find(std::make_pair(dev, stream));
  if (it == g_ws.end() && !info.scratch_zeroed) return TOPK_SUCCESS;
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  if (it != g_ws.end()) {
    topk_status_t st = take_fault(page_word(info, it->second.fault_word), &it->second.reported);
    if (st != TOPK_SUCCESS) return st;
  }
  if (info.scratch_zeroed) {
    // the scratch's count from the device itself (no page may exist yet)
    uint32_t count = 0;
    e = hipMemcpy(&count, info.scratch + topk::kHdrFaultCount, sizeof(uint32_t), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy");
    return take_fault(count, &info.scratch_reported);
  }
  return TOPK_SUCCESS;
}

topk_status_t topk_set_wait_limit(uint32_t polls) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_spin_limit = polls == 0u ? topk::kDefaultSpinLimit : polls;
  return TOPK_SUCCESS;
}

topk_status_t topk_set_scratch_limit(uint64_t words) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_scratch_limit = (size_t)words;
  return TOPK_SUCCESS;
}

int32_t topk_abi_version(void) { return 5; }

}  // extern "C"
