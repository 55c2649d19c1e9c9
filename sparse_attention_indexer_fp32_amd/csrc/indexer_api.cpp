// C-ABI layer of the indexer scoring and the fused scoring + exact top-k:
// argument and device checks, the launch shape (workgroups of 8 query rows;
// the key range split into windows when there are too few row blocks to fill
// the device), and the per-(device, stream) candidate buffers.  The exact
// select over the packed candidates is topk_transform with the candidates'
// positions as a page table of page size 1, so its output is the positions.

#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "indexer_internal.h"
#include "indexer_topk.h"
#include "topk_internal.h"

namespace {

struct Buffers {
  void* ptr = nullptr;
  size_t bytes = 0;
};

std::mutex& g_mu = topk::lib_mutex();   // the library's one lock
std::map<int, int> g_cus;                                   // device -> CUs (gfx950 only)
std::map<std::pair<int, hipStream_t>, Buffers> g_bufs;
int64_t g_window_override = 0;                              // 0: automatic
int g_select_mode = -1;                                     // indexer_topk: -1 automatic, 0 fused, 1 dense

topk_status_t fail(topk_status_t st, const std::string& msg) {
  topk::set_last_error(msg.c_str());
  return st;
}

topk_status_t hip_fail(hipError_t e, const char* what) {
  return fail(TOPK_ERROR_LAUNCH, std::string(what) + ": " + hipGetErrorString(e));
}

// Caller holds g_mu.  CUs of the current device, or 0 when it is not gfx950.
topk_status_t device_cus(int* dev_out, int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  *dev_out = dev;
  auto it = g_cus.find(dev);
  if (it == g_cus.end()) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    it = g_cus.emplace(dev, ok ? prop.multiProcessorCount : 0).first;
    if (!ok) return fail(TOPK_ERROR_UNSUPPORTED, std::string("device ") + prop.gcnArchName + " is not gfx950");
  }
  if (it->second == 0) return fail(TOPK_ERROR_UNSUPPORTED, "device is not gfx950");
  *cus = it->second;
  return TOPK_SUCCESS;
}

// Caller holds g_mu.
topk_status_t get_buffers(int dev, hipStream_t stream, size_t bytes, void** ptr) {
  Buffers& b = g_bufs[std::make_pair(dev, stream)];
  if (b.ptr && b.bytes >= bytes) {
    *ptr = b.ptr;
    return TOPK_SUCCESS;
  }
  void* p = nullptr;
  hipError_t e = hipMalloc(&p, bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(TOPK_ERROR_OUT_OF_MEMORY, std::string("indexer buffers hipMalloc: ") + hipGetErrorString(e));
  }
  // the smaller buffer stays allocated until topk_release_workspaces: work
  // queued on it (or a graph captured with it) may still use it
  topk::retire_buffer(b.ptr);
  b.ptr = p;
  b.bytes = bytes;
  *ptr = p;
  return TOPK_SUCCESS;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Windows over [0, num_kv): enough (row block, window) workgroups for two per
// CU, windows of at least 2048 positions, a multiple of 64 each (the kernels
// stage 64 positions at a time and must not cross a window's edge).
void plan_windows(int64_t num_q, int64_t num_kv, int cus, int32_t* nwin, int64_t* window) {
  if (g_window_override > 0) {
    *window = g_window_override;
    *nwin = (int32_t)ceil_div(num_kv > 0 ? num_kv : 1, g_window_override);
    return;
  }
  const int64_t blocks = ceil_div(num_q, indexer::rows_per_workgroup());
  int64_t n = ceil_div(2 * (int64_t)cus, blocks);
  const int64_t most = ceil_div(num_kv, 2048);
  if (n > most) n = most;
  if (n < 1) n = 1;
  int64_t w = ceil_div(ceil_div(num_kv, n), 64) * 64;
  if (w < 64) w = 64;
  *window = w;
  *nwin = (int32_t)ceil_div(num_kv > 0 ? num_kv : 1, w);
}

topk_status_t check_common(const uint8_t* q, const float* weights, const uint8_t* kv, const float* kv_scale,
                           const int32_t* ks, const int32_t* ke, int32_t num_q, int64_t num_kv) {
  if (num_q < 0 || num_kv < 0) return fail(TOPK_ERROR_INVALID_VALUE, "num_q and num_kv must be >= 0");
  if (num_kv > (int64_t)INT32_MAX) return fail(TOPK_ERROR_INVALID_VALUE, "num_kv must fit in int32");
  if (num_q == 0) return TOPK_SUCCESS;
  if (!q || !weights || !ks || !ke) return fail(TOPK_ERROR_INVALID_VALUE, "q, weights, ks and ke must be non-null");
  if (num_kv > 0 && (!kv || !kv_scale))
    return fail(TOPK_ERROR_INVALID_VALUE, "kv and kv_scale must be non-null when num_kv > 0");
  if ((reinterpret_cast<uintptr_t>(kv) & 15) != 0 || (reinterpret_cast<uintptr_t>(q) & 15) != 0)
    return fail(TOPK_ERROR_INVALID_VALUE, "q and kv must be 16-byte aligned");
  return TOPK_SUCCESS;
}

}  // namespace

namespace indexer {

// Both are called with the library lock held (topk_release_workspaces).
bool has_buffers() { return !g_bufs.empty(); }

void release_buffers() {
  for (auto& kv : g_bufs)
    if (kv.second.ptr) (void)hipFree(kv.second.ptr);
  g_bufs.clear();
}

}  // namespace indexer

extern "C" {

topk_status_t indexer_logits(const uint8_t* q, const float* weights, const uint8_t* kv, const float* kv_scale,
                             const int32_t* ks, const int32_t* ke, float* logits, hipStream_t stream,
                             int32_t num_q, int64_t num_kv, int64_t logits_stride) {
  topk::set_last_error("");
  topk_status_t st = check_common(q, weights, kv, kv_scale, ks, ke, num_q, num_kv);
  if (st != TOPK_SUCCESS) return st;
  if (logits_stride < 0) return fail(TOPK_ERROR_INVALID_VALUE, "logits_stride must be >= 0");
  if (num_q == 0) return TOPK_SUCCESS;
  if (!logits && logits_stride > 0) return fail(TOPK_ERROR_INVALID_VALUE, "logits must be non-null");
  std::lock_guard<std::mutex> lock(g_mu);
  int dev = 0, cus = 0;
  st = device_cus(&dev, &cus);
  if (st != TOPK_SUCCESS) return st;
  if (num_kv == 0 || logits_stride == 0) return TOPK_SUCCESS;
  indexer::ScanArgs a{};
  a.q = q;
  a.weights = weights;
  a.kv = kv;
  a.kv_scale = kv_scale;
  a.ks = ks;
  a.ke = ke;
  a.num_q = num_q;
  a.num_kv = num_kv;
  plan_windows(num_q, num_kv, cus, &a.nwin, &a.window);
  a.logits = logits;
  a.logits_stride = logits_stride;
  hipError_t e = indexer::launch_logits(a, a.nwin, stream);
  if (e != hipSuccess) return hip_fail(e, "indexer logits launch");
  char buf[160];
  std::snprintf(buf, sizeof(buf), "indexer-logits grid=%lldx%d window=%lld",
                (long long)ceil_div(num_q, indexer::rows_per_workgroup()), a.nwin, (long long)a.window);
  topk::set_last_launch(buf);
  return TOPK_SUCCESS;
}

topk_status_t indexer_topk(const uint8_t* q, const float* weights, const uint8_t* kv, const float* kv_scale,
                           const int32_t* ks, const int32_t* ke, int32_t k, int32_t* out_idx, hipStream_t stream,
                           int32_t num_q, int64_t num_kv) {
  topk::set_last_error("");
  if (k < 1 || k > TOPK_MAX_K) return fail(TOPK_ERROR_INVALID_VALUE, "k must be in [1, 2048]");
  topk_status_t st = check_common(q, weights, kv, kv_scale, ks, ke, num_q, num_kv);
  if (st != TOPK_SUCCESS) return st;
  if (num_q == 0) return TOPK_SUCCESS;
  if (!out_idx) return fail(TOPK_ERROR_INVALID_VALUE, "out_idx must be non-null");
  indexer::ScanArgs a{};
  int64_t row_cap = 0;
  // The lock is held from the scan launch through the select's launch, so no
  // other call can queue work on this stream's candidate buffers in between.
  std::lock_guard<std::mutex> lock(g_mu);
  int dev = 0, cus = 0;
  st = device_cus(&dev, &cus);
  if (st != TOPK_SUCCESS) return st;
  a.q = q;
  a.weights = weights;
  a.kv = kv;
  a.kv_scale = kv_scale;
  a.ks = ks;
  a.ke = ke;
  a.num_q = num_q;
  a.num_kv = num_kv;
  a.k = k;
  plan_windows(num_q, num_kv, cus, &a.nwin, &a.window);
  // Windows shorter than kDenseWindowRatio x k: every window keeps at least k
  // of its positions, and the fused scan's list work costs more than writing
  // every score and selecting from the buffer (MI355X, causal prefills: 16K
  // windows at k 2048 fused 1.16 ms against dense 0.60 ms; 64K windows at
  // k 2048 2.64-2.77 against 2.19-2.23 ms; 16K windows at k 512 1.47
  // against 1.01 ms).  Those calls score densely into a buffer (up to
  // kDenseMaxBytes) and select from it.  Longer windows (the 262144-key
  // prefill: 17.3 against 16.9 ms, a 8.6 GB buffer) keep the fused scan.
  constexpr int64_t kDenseWindowRatio = 64;
  constexpr double kDenseMaxBytes = 8.0 * (1ull << 30);
  const bool dense = g_select_mode == 1 ||
                     (g_select_mode < 0 && (int64_t)k * kDenseWindowRatio > a.window &&
                      (double)num_q * (double)num_kv * 4.0 <= kDenseMaxBytes);
  if (dense) {
    const int64_t width = num_kv;   // score rows' stride: no clamped range is longer
    const size_t scores = (size_t)num_q * (size_t)width;
    const size_t bytes = scores * 4 + (size_t)num_q * 4 + (size_t)num_q * (size_t)k * 4 + 256;
    void* base = nullptr;
    st = get_buffers(dev, stream, bytes, &base);
    if (st != TOPK_SUCCESS) return st;
    char* p = static_cast<char*>(base);
    float* sc = reinterpret_cast<float*>(p);
    p += scores * 4;
    int32_t* len = reinterpret_cast<int32_t*>(p);
    p += (size_t)num_q * 4;
    int32_t* rel = reinterpret_cast<int32_t*>(p);
    a.logits = sc;
    a.logits_stride = width;
    hipError_t e = indexer::launch_logits(a, a.nwin, stream);
    if (e == hipSuccess) e = indexer::launch_row_lengths(a, len, stream);
    if (e != hipSuccess) return hip_fail(e, "indexer dense launch");
    // row-relative positions through out_raw (no page table: out_idx gets -1
    // from the select and is then overwritten with the absolute positions)
    st = topk::transform_locked(sc, len, nullptr, k, 1, out_idx, rel, stream, num_q, width, 0);
    if (st != TOPK_SUCCESS) return st;
    e = indexer::launch_absolute_positions(a, rel, out_idx, stream);
    if (e != hipSuccess) return hip_fail(e, "indexer position launch");
    char buf[200];
    std::snprintf(buf, sizeof(buf), "indexer-topk dense grid=%lldx%d window=%lld + select %s",
                  (long long)ceil_div(num_q, indexer::rows_per_workgroup()), a.nwin, (long long)a.window,
                  topk_last_launch());
    topk::set_last_launch(buf);
    return TOPK_SUCCESS;
  }
  // a list never holds more than its window; a capacity below the window
  // leaves room for k entries plus a tile after every trim
  int64_t cap = 4 * (int64_t)k > 4096 ? 4 * (int64_t)k : 4096;
  if (cap > a.window) cap = a.window;
  a.cap = (int32_t)cap;
  // With one window per row the select reads the lists in place (no final
  // trim, no packed copy): every list entry is a candidate, and the list holds
  // a top-k of its row.
  a.inplace = a.nwin == 1 ? 1 : 0;
  row_cap = a.inplace ? 0 : (int64_t)a.nwin * k;
  a.row_cap = row_cap;
  const size_t lists = (size_t)num_q * a.nwin * (size_t)cap;
  const size_t packed = (size_t)num_q * (size_t)row_cap;
  const size_t bytes = lists * 8 + packed * 8 + (size_t)num_q * 4 + 256;
  void* base = nullptr;
  st = get_buffers(dev, stream, bytes, &base);
  if (st != TOPK_SUCCESS) return st;
  char* p = static_cast<char*>(base);
  a.cand_score = reinterpret_cast<float*>(p);
  p += lists * 4;
  a.cand_pos = reinterpret_cast<int32_t*>(p);
  p += lists * 4;
  a.row_score = reinterpret_cast<float*>(p);
  p += packed * 4;
  a.row_pos = reinterpret_cast<int32_t*>(p);
  p += packed * 4;
  a.row_count = reinterpret_cast<int32_t*>(p);
  hipError_t e = indexer::launch_scan(a, a.nwin, stream);
  if (e != hipSuccess) return hip_fail(e, "indexer scan launch");
  // exact select over the candidates (the lists in place, or their packed
  // copies); the positions act as a page table of page size 1, so out_idx
  // receives them directly
  if (a.inplace)
    st = topk::transform_locked(a.cand_score, a.row_count, a.cand_pos, k, 1, out_idx, nullptr, stream, num_q, cap,
                                cap);
  else
    st = topk::transform_locked(a.row_score, a.row_count, a.row_pos, k, 1, out_idx, nullptr, stream, num_q, row_cap,
                                row_cap);
  if (st != TOPK_SUCCESS) return st;
  char buf[200];
  std::snprintf(buf, sizeof(buf), "indexer-topk grid=%lldx%d window=%lld cap=%d%s + select %s",
                (long long)ceil_div(num_q, indexer::rows_per_workgroup()), a.nwin, (long long)a.window, a.cap,
                a.inplace ? " in-place" : "", topk_last_launch());
  topk::set_last_launch(buf);
  return TOPK_SUCCESS;
}

topk_status_t indexer_set_select_mode(int32_t mode) {
  if (mode < -1 || mode > 1) return fail(TOPK_ERROR_INVALID_VALUE, "mode must be -1 (automatic), 0 or 1");
  std::lock_guard<std::mutex> lock(g_mu);
  g_select_mode = mode;
  return TOPK_SUCCESS;
}

topk_status_t indexer_set_window_override(int64_t window) {
  if (window < 0 || window % 64 != 0 || window > (int64_t)INT32_MAX)
    return fail(TOPK_ERROR_INVALID_VALUE, "window must be 0 or a positive multiple of 64");
  std::lock_guard<std::mutex> lock(g_mu);
  g_window_override = window;
  return TOPK_SUCCESS;
}

}  // extern "C"
