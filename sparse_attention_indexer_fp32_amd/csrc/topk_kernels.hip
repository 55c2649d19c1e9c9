// gfx950 (CDNA4) kernels: exact per-row top-k over fp32 scores, fused with
// the KV page-table transform.
//
// The method is an MSB-first radix select on an order-preserving integer key
// (flash-float-jit-kernels README, method bullets: per-block parallel
// histograms, a prefix sum over the bins to find the threshold bin, a monotone
// bin map so bin(x) >= bin(y) implies x >= y), with the page transform done as
// a separate pass over the selected raw positions (SGLang PR #26788 commit
// notes: write raw indices, barrier, then gather + transform).
//
// CDNA4 shape of it:
//   * A workgroup of 1024 threads (16 wave64s) keeps its share of a row in
//     VGPRs: E keys per thread, loaded once from HBM with dwordx4 loads.
//     Every radix pass re-reads registers, never HBM.
//   * Digits: 12 bits (4096 bins), then 10 and 10.  Each pass builds an LDS
//     histogram of the keys that still match the threshold prefix, then a
//     workgroup scan (wave64 shuffle scan + per-wave totals in LDS) finds the
//     bin where the count from the top crosses the remaining k.
//   * Long rows are split over G workgroups (there is no distributed shared
//     memory on CDNA4): partial histograms are merged with agent-scope global
//     atomics and a per-row barrier in global memory (the grid is sized to
//     what the GPU holds resident, so every workgroup of a row is running).  When the threshold bin
//     is small enough, each workgroup appends its threshold-bin elements to a
//     global candidate list and the last workgroup to leave the row finishes
//     the remaining digits on the candidates in LDS -- one barrier per row
//     instead of one per digit.
//   * Selected positions go to a staging list in LDS; after a barrier one
//     pass gathers the page-table entries and writes out_idx / out_raw, -1
//     padded.  A split row's workgroups each write the slots their own keys
//     took (one batched gather per workgroup), and the finisher only the
//     slots it fills from the candidates.
//   * When more rows than slots fit resident, rows cycle over the slots; in
//     that launch a row that fits one workgroup runs in one workgroup of its
//     slot, with no cross-workgroup merge.
//   * Large batches stream instead (stream_rows_kernel): one workgroup per
//     row, a gate set from a sample of the row, the keys at or above it
//     appended to an LDS candidate list while the rest of the row streams
//     past in register-held chunks (two or three in flight); the radix
//     digits then run on the list.  Rows past the grid come from a ticket
//     queue.
//   * A row's scores are read once, with non-temporal loads; only the
//     fallback re-stream and the sorted finish read a row again.
//   * The deterministic entry point adds a second launch (sorted_rows_kernel)
//     that puts each row's selection in the plain definition's order.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "topk_internal.h"

namespace topk {
namespace {

enum Mode : int { kModeNone = 0, kModeTakeAll = 1, kModeTies = 2, kModeCands = 3 };

// fp32 -> uint32 whose unsigned order is the value order (-0.0 just below +0.0).
// Key 0 belongs only to the NaN pattern 0xFFFFFFFF, so 0 marks "no element".
__device__ __forceinline__ uint32_t order_key_bits(uint32_t u) {
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Word 3 of a CDNA (gfx9-family) raw buffer descriptor: 32-bit data format,
// no swizzle; loads past num_records return zero.
constexpr int kBufferWord3 = 0x00020000;

// Cache-policy operand of the buffer loads (gfx950: bit 1 = nt, non-temporal).
constexpr int kLoadStream = 2;
constexpr int kLoadReuse = 0;

// The thread index through an empty asm, so values derived from it are
// recomputed where they are used instead of being hoisted out of the row loop
// (LICM would otherwise keep dozens of per-element addresses live in VGPRs).
__device__ __forceinline__ int opaque_tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Marks register-resident keys as redefined, so per-key digits and LDS
// addresses are computed inside each radix pass rather than hoisted out of
// the pass loop (which would keep several values per key live at once).
template <int E>
__device__ __forceinline__ void launder(uint32_t (&key)[E]) {
#pragma unroll
  for (int j = 0; j < E; ++j) asm volatile("" : "+v"(key[j]));
}

// A workgroup-uniform value read from LDS (or loaded from a uniform address),
// declared uniform so control flow that depends on it stays scalar.
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// p[i] at a wave-uniform index, read through the scalar data cache (only for
// arrays that nothing writes while the kernel runs, such as the row lengths:
// that cache is not kept coherent within a launch): the read waits on the
// scalar counter, not behind vector loads issued before it.
__device__ __forceinline__ int32_t scalar_read(const int32_t* p, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}

// ---- agent-scope (whole-GPU, across XCDs) memory operations ----------------
__device__ __forceinline__ void g_add(uint32_t* p, uint32_t v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t g_add_ret(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t g_add64_ret(uint64_t* p, uint64_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wrapping increment: returns the old value and stores old + 1, or 0 once the
// old value has reached `last` (one atomic; the counter resets itself).
__device__ __forceinline__ uint32_t g_inc_wrap(uint32_t* p, uint32_t last) {
  return __builtin_amdgcn_atomic_inc32(p, last, __ATOMIC_RELAXED, "agent");
}
// A row-queue ticket (one lane asks).  The address is made per-lane for the
// compiler (it is the same word): an atomic on a wave-uniform address is
// rewritten into one per wave whose result is read back at once, and that
// read waits for every load the wave has in flight.
__device__ __forceinline__ uint32_t take_ticket(uint32_t* queue) {
  return g_add_ret(queue + ((uint32_t)opaque_tid() >> 16), 1u);
}
__device__ __forceinline__ uint32_t g_load(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void g_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- scans -----------------------------------------------------------------
// DPP controls (gfx9 family).
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

// Inclusive sum over the 16 lanes of each DPP row (lane 15 of a row ends with
// the row total).  Out-of-row sources read as 0.
__device__ __forceinline__ uint32_t row16_inclusive_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr1, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr2, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr4, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr8, 0xf, 0xf, false);
  return v;
}

// Inclusive sum over the 64 lanes of a wave: per-row scans, then the row
// totals carried across rows with the row-broadcast DPP modes.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v, int tid) {
  (void)tid;
  v = row16_inclusive_scan(v);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowBcast15, 0xa, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowBcast31, 0xc, 0xf, false);
  return v;
}

// Exclusive scan over an NT-thread workgroup in thread order; `total` gets
// the sum.  sh_scan needs NT/64 + 1 words.  Contains barriers: call uniformly.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* sh_scan, uint32_t& total,
                                                        int tid) {
  constexpr int kW = NT / 64;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const uint32_t inc = wave_inclusive_scan(v, tid);
  if (lane == 63) sh_scan[wid] = inc;
  __syncthreads();
  if (wid == 0) {
    const uint32_t w = lane < kW ? sh_scan[lane] : 0u;
    const uint32_t wi = wave_inclusive_scan(w, tid);
    if (lane < kW) sh_scan[lane] = wi - w;
    if (lane == kW - 1) sh_scan[kW] = wi;
  }
  __syncthreads();
  const uint32_t r = sh_scan[wid] + inc - v;
  total = sh_scan[kW];
  __syncthreads();
  return r;
}

// Threshold bin of histogram h[0, NB), NB = 4096, 2048 or 1024: the highest bin t
// with sum_{b >= t} h[b] >= need.  Writes sh_var[0] = t, sh_var[1] = count in
// bins above t, sh_var[2] = h[t].  (If the histogram holds fewer than `need`
// elements -- impossible for valid input -- it reports bin 0 with counts 0.)
//
// Two levels, one barrier in between: every group of 64 bins is summed (each
// of the NT threads sums NB/NT bins, then a DPP row scan or a lane butterfly
// adds up the threads of a group) into sh_coarse; then wave 0 scans the group
// totals from the top to find the crossing group, and scans that group's 64
// bins to find the crossing bin (ballot + first set lane locate both).
template <int NT, int NB>
__device__ __forceinline__ void find_threshold(const uint32_t* h, uint32_t need, uint32_t* sh_coarse,
                                               uint32_t* sh_var, int tid) {
  constexpr int kPer = NB / NT;           // bins per thread
  constexpr int kTpg = 64 / kPer;         // threads per 64-bin group
  constexpr int ngroups = NB / 64;
  const int lane = tid & 63;
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) sum += h[tid * kPer + i];
  if (kTpg == 16) {
    sum = row16_inclusive_scan(sum);
  } else if (kTpg == 64) {
    sum = wave_inclusive_scan(sum, tid);
  } else {
#pragma unroll
    for (int d = 1; d < kTpg; d <<= 1) sum += __shfl_xor(sum, d, 64);
  }
  if ((tid % kTpg) == (kTpg == 16 || kTpg == 64 ? kTpg - 1 : 0)) sh_coarse[tid / kTpg] = sum;
  __syncthreads();
  if (tid < 64) {
    const uint32_t v = lane < ngroups ? sh_coarse[ngroups - 1 - lane] : 0u;   // lane 0 = highest group
    const uint32_t cum = wave_inclusive_scan(v, tid);
    const uint64_t hit = __ballot(lane < ngroups && cum >= need);
    uint32_t bin = 0, above = 0, cnt = 0;
    if (hit != 0ull) {
      const int lg = __builtin_ctzll(hit);
      const int grp = ngroups - 1 - lg;
      const uint32_t before = (uint32_t)__builtin_amdgcn_readlane((int)cum, lg) -
                              (uint32_t)__builtin_amdgcn_readlane((int)v, lg);
      const uint32_t fv = h[grp * 64 + 63 - lane];                         // lane 0 = highest bin of the group
      const uint32_t fcum = wave_inclusive_scan(fv, tid);
      const uint64_t fhit = __ballot(before + fcum >= need);
      const int lf = __builtin_ctzll(fhit);
      bin = (uint32_t)(grp * 64 + 63 - lf);
      cnt = (uint32_t)__builtin_amdgcn_readlane((int)fv, lf);
      above = before + (uint32_t)__builtin_amdgcn_readlane((int)fcum, lf) - cnt;
    }
    if (lane == 0) {
      sh_var[0] = bin;
      sh_var[1] = above;
      sh_var[2] = cnt;
    }
  }
  __syncthreads();
}

// Waits until this wave's outstanding memory operations have completed.  All
// cross-workgroup data moves through agent-scope atomics and agent-scope
// (sc1, coherent) loads and stores, so once a wave's operations are complete
// they are visible to every XCD; no L2 write-back or invalidate is needed.
__device__ __forceinline__ void wave_mem_drain() { __builtin_amdgcn_s_waitcnt(0); }

// Per-row barrier among the G workgroups of one slot.  The grid never exceeds
// the device's resident-workgroup capacity, so all G are normally running at
// once (a kernel that holds CUs on another stream can break that: there is no
// cooperative launch).  Workgroup g arrives on its group's counter; the last
// of a group arrives on the top counter; the last group's closer publishes
// the next generation.  Arrivals are wrapping increments, so the last one on
// a counter also resets it to zero in the same atomic: every counter is zero
// again before the publication (which follows the top counter's last
// arrival, which follows each group's), and the barrier resets itself across
// calls and graph replays with no reset stores to drain.  Each workgroup
// drains its own writes before it arrives.  Each workgroup tracks the
// generation it waits for in `gen` (read once per launch: no barrier of the
// slot can complete before this workgroup has arrived, so the value is stable
// until then).
//
// The wait is bounded by `spin_limit` polls.  A wait that gives up sets the
// fault word and `gave_up`; every other wait that sees the fault word set gives
// up too, so the kernel always drains.  The launch's outputs are then invalid:
// its last workgroup out puts the workspace back in its initial state (fault
// word included) and counts the fault for the host (launch_exit), so the next
// launch starts clean and waits its full limit.
__device__ __forceinline__ void row_barrier(uint32_t* bar, int G, int g, uint32_t& gen, uint32_t* fault,
                                            uint32_t spin_limit, uint32_t& gave_up, int tid) {
  wave_mem_drain();
  __syncthreads();
  if (tid == 0) {
    ++gen;
    const int grp = g / kBarGroup;
    const int ngroups = (G + kBarGroup - 1) / kBarGroup;
    const uint32_t gsize = (uint32_t)(G - grp * kBarGroup < kBarGroup ? G - grp * kBarGroup : kBarGroup);
    // Wrapping increments: a counter's last arrival sees gsize - 1 (ngroups
    // - 1) and leaves it at 0 in the same atomic, so every counter is zero
    // again before the generation that releases the workgroups is published.
    bool closer = false;
    if (g_inc_wrap(bar + (size_t)grp * kBarLine, gsize - 1u) == gsize - 1u)
      closer = ngroups == 1 || g_inc_wrap(bar + kBarTop, (uint32_t)ngroups - 1u) == (uint32_t)ngroups - 1u;
    if (closer) {
      g_store(bar + kBarGen, gen);   // nothing this workgroup does next depends on its completion
    } else {
      uint32_t spins = 0;
      while ((int32_t)(g_load(bar + kBarGen) - gen) < 0) {
        if (spins >= spin_limit || ((spins & 1023u) == 1023u && g_load(fault) != 0u)) {
          g_store(fault, 1u);
          gave_up = 1u;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        ++spins;
      }
      wave_mem_drain();
    }
  }
  __syncthreads();
}

// Arrivals on the launch-exit counter carry this much per wait given up.
constexpr uint32_t kExitFaultUnit = 1u << 16;

// End of a split-row launch, called by every workgroup once it has no more
// rows.  Each workgroup counts itself out (plus kExitFaultUnit if one of its
// waits gave up); its last workspace writes other than zeroes were drained at
// its last row's exit, so the arrival needs no drain of its own.  The last
// workgroup out resets the counter.  If any wait of the launch gave up, it
// first zeroes every barrier block and region and the fault word -- a barrier
// that gave up can leave stray arrivals and partial histograms behind -- and
// counts the fault in the header and in the host-visible word.  Uniform;
// contains barriers.
__device__ __forceinline__ void launch_exit(const KernelArgs& a, uint32_t gave_up, uint32_t* sh_flag, int tid) {
  __syncthreads();
  if (tid == 0) {
    const uint32_t mine = 1u + (gave_up != 0u ? kExitFaultUnit : 0u);
    const uint32_t before = g_add_ret(a.ws + kHdrLaunchExit, mine);
    const bool last = (before & (kExitFaultUnit - 1u)) == gridDim.x - 1u;
    const uint32_t faults = (before >> 16) + (gave_up != 0u ? 1u : 0u);
    *sh_flag = last ? (faults != 0u ? 2u : 1u) : 0u;
  }
  __syncthreads();
  const uint32_t flag = uniform(*sh_flag);
  if (flag == 0u) return;
  if (flag == 2u) {
    const size_t words = (size_t)a.ws_slots * kBarWords + (size_t)a.ws_slots * 2 * kRegionWords;
    for (size_t i = (size_t)tid; i < words; i += kThreads) g_store(a.ws + kHdrWords + i, 0u);
    if (tid == 0) {
      g_store(a.ws + kHdrFault, 0u);
      const uint32_t count = g_add_ret(a.ws + kHdrFaultCount, 1u) + 1u;
      if (a.fault_host != nullptr)
        __hip_atomic_store(a.fault_host, count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
  if (tid == 0) g_store(a.ws + kHdrLaunchExit, 0u);
}

// Gather + transform pass: slot j < n holds raw position r (trivial rows: r = j);
// out = page_table[row, r >> log2_page] << log2_page | (r & (page_size - 1)).
// Slots past n, and any r outside [0, L), give -1.  `pt_row` is the row's
// page table, in global memory or an LDS copy of it.  Writes slots [from, k).
template <int NT>
__device__ __forceinline__ void write_row_output(const KernelArgs& a, int64_t row, int64_t L, int n, bool trivial,
                                                 const int32_t* sh_raw, int tid, const int32_t* pt_row = nullptr,
                                                 int from = 0) {
  const int k = a.k;
  const int s = a.log2_page;
  const uint32_t pmask = (1u << s) - 1u;
  int32_t* o = a.out + row * (int64_t)k;
  int32_t* orw = a.out_raw ? a.out_raw + row * (int64_t)k : nullptr;
  const int32_t* pt = pt_row != nullptr ? pt_row : a.page_table + row * a.pages_per_row;
  for (int j = from + tid; j < k; j += NT) {
    int32_t r = -1;
    if (j < n) r = trivial ? j : sh_raw[j];
    int32_t v = -1;
    if (r >= 0 && (int64_t)r < L) {
      const int64_t pg = (int64_t)(r >> s);
      if (pg < a.pages_per_row) v = (int32_t)(((uint32_t)pt[pg] << s) | ((uint32_t)r & pmask));
    } else {
      r = -1;
    }
    o[j] = v;
    if (orw) orw[j] = r;
  }
}

// Position r of the row (in [0, L)) straight to output slot j, through the
// same transform as write_row_output.  Split rows: each workgroup writes the
// slots its own keys took, so no workgroup gathers the whole row's output.
__device__ __forceinline__ void write_slot(const KernelArgs& a, int64_t row, uint32_t j, int32_t r) {
  const int s = a.log2_page;
  const int64_t pg = (int64_t)(r >> s);
  int32_t v = -1;
  if (pg < a.pages_per_row)
    v = (int32_t)(((uint32_t)a.page_table[row * a.pages_per_row + pg] << s) | ((uint32_t)r & ((1u << s) - 1u)));
  a.out[row * (int64_t)a.k + j] = v;
  if (a.out_raw) a.out_raw[row * (int64_t)a.k + j] = r;
}

// Records how a row's selection ended, for the sorted finish: every key x of
// the row with x >= floor and (x >> shift) > prefix was selected, and `need`
// of the `cnt` with (x >> shift) == prefix.  When cnt == need (the bin is not
// cut) the selected set is the canonical one, whatever the order.  shift 32
// with floor 0 and prefix 0 selects every position below the row's length
// (rows with L <= k).  Called by one thread.
// `keys`: the row's selected keys were also written to a.sel_key.
__device__ __forceinline__ void record_selection(const KernelArgs& a, int64_t row, uint32_t prefix, int shift,
                                                 uint32_t need, uint32_t cnt, uint32_t floor, bool keys = false) {
  if (a.meta == nullptr) return;
  uint32_t* m = a.meta + row * kMetaWords;
  m[0] = prefix;
  m[1] = (uint32_t)shift;
  m[2] = need;
  m[3] = floor;
  m[4] = cnt != need ? 1u : 0u;
  m[5] = keys ? 1u : 0u;
}

// Histogram of one radix digit over the register-resident keys that match the
// prefix of the previous digits.
// Register slots per thread that form the pass-0 sample (see hist_pass0).
template <int E>
struct SampleSlots {
  static constexpr int value = E >= 16 ? 8 : E;
};

// Pass-0 histogram of the register-resident keys.  Slots [0, S) of every
// thread are a sample: its full histogram gives the highest bin t_s such that
// at least `need` sampled keys lie at or above it.  The row then has at least
// `need` keys at or above t_s, so the threshold bin is >= t_s and only bins
// >= t_s need exact counts: the other slots add to the histogram only when
// their bin is >= t_s.  Exact for every bin the threshold search can reach,
// with several times fewer LDS atomics on the usual (non-adversarial) rows.
// For a split row each workgroup gates on its own sample, which is as valid:
// the row's threshold bin is >= every workgroup's t_s.
template <int E>
// Returns t_s (the lowest bin the row's threshold can be in, as far as this
// workgroup's keys tell); with `want_gate` false and no sampling, returns 0
// without searching.
__device__ __forceinline__ uint32_t hist_pass0(const uint32_t (&key)[E], uint32_t need, uint32_t* h,
                                               uint32_t* sh_scan, uint32_t* sh_var, int tid, bool want_gate) {
  constexpr int S = SampleSlots<E>::value;
#pragma unroll
  for (int j = 0; j < S; ++j)
    if (key[j]) atomicAdd(&h[key[j] >> 20], 1u);
  if (S == E && !want_gate) return 0u;
  __syncthreads();
  find_threshold<kThreads, kBinsWide>(h, need, sh_scan, sh_var, tid);
  const uint32_t ts = uniform(sh_var[0]);
  if (S == E) return ts;
  // Bin >= 1 also excludes key 0 (no element).
  const uint32_t gate = ts > 1u ? ts : 1u;
#pragma unroll
  for (int j = S; j < E; ++j)
    if ((key[j] >> 20) >= gate) atomicAdd(&h[key[j] >> 20], 1u);
  return ts;
}

template <int E>
__device__ __forceinline__ void hist_resident(const uint32_t (&key)[E], int pass, uint32_t prefix,
                                              uint32_t* h) {
  if (pass == 0) {
#pragma unroll
    for (int j = 0; j < E; ++j)
      if (key[j]) atomicAdd(&h[key[j] >> 20], 1u);
  } else if (pass == 1) {
#pragma unroll
    for (int j = 0; j < E; ++j)
      if ((key[j] >> 20) == prefix) atomicAdd(&h[(key[j] >> 10) & 1023u], 1u);
  } else {
#pragma unroll
    for (int j = 0; j < E; ++j)
      if ((key[j] >> 10) == prefix) atomicAdd(&h[key[j] & 1023u], 1u);
  }
}

// Among the candidates whose key equals `key`, finds the `need` (< their
// count) with the lowest positions, by an MSB-first radix select on v =
// ~position (the largest v are the lowest positions; positions are distinct,
// so it ends with exactly `need`): on return exactly those members have
// (v >> vshift) >= vprefix.  Digits of 11, 11 and 10 bits, so sh_hist needs
// 2048 words.  Contains barriers: call uniformly.
template <int NT>
__device__ void lowest_positions(int ncand, uint32_t key, uint32_t need, const uint32_t* sh_ckey,
                                 const int32_t* sh_cpos, uint32_t* sh_hist, uint32_t* sh_scan, uint32_t* sh_var,
                                 int tid, uint32_t& vprefix, int& vshift) {
  vprefix = 0;
  vshift = 32;
  uint32_t vneed = need;
  for (int level = 0; level < 3; ++level) {
    const int dshift = level == 0 ? 21 : (level == 1 ? 10 : 0);
    const uint32_t mask = level == 2 ? 1023u : 2047u;
    for (int b = tid; b < 2048; b += NT) sh_hist[b] = 0;
    __syncthreads();
    for (int i = tid; i < ncand; i += NT) {
      if (sh_ckey[i] != key) continue;
      const uint32_t v = ~(uint32_t)sh_cpos[i];
      if (vshift >= 32 || (v >> vshift) == vprefix) atomicAdd(&sh_hist[(v >> dshift) & mask], 1u);
    }
    __syncthreads();
    if (level == 2) find_threshold<NT, kBinsNarrow>(sh_hist, vneed, sh_scan, sh_var, tid);
    else find_threshold<NT, 2048>(sh_hist, vneed, sh_scan, sh_var, tid);
    const uint32_t bin = uniform(sh_var[0]), gtc = uniform(sh_var[1]), cnt = uniform(sh_var[2]);
    vneed -= gtc;
    vprefix = level == 0 ? bin : ((vprefix << (level == 1 ? 11 : 10)) | bin);
    vshift = dshift;
    if (cnt == vneed) break;
  }
}

// Finishes a row from candidates held in LDS.  (prefix, shift) name the
// current threshold bin (the candidates' keys >> shift), `cnt` how many keys
// it holds and `need` how many of its keys are still to be selected; the
// candidates contain every key of the threshold bin, and may also hold keys
// above it (those are selected outright).  Refines the bin with the remaining
// 10-bit digits, then writes the strictly-greater keys to slots
// [gt_base, n - need_final) and `need_final` keys of the final bin to
// [n - need_final, n).
// On return (prefix, shift, cnt, need) describe the final bin: every
// candidate with (key >> shift) == prefix is of it, cnt of them, `need` of
// them were selected.
// With `fill`, slots [0, n) of sh_raw are first set to -1 (nothing else
// has written them yet).  With INDEX the slots receive candidate indices
// (into sh_ckey / sh_cpos) instead of positions.  With `key_out` (global
// memory, the row's k slots) each slot's key is written there too.  With
// `canon`, a final bin that has to be cut (equal keys, more than `need` of
// them) gives its `need` lowest positions, the plain definition's choice,
// and `cnt` returns equal to `need`: the selected set is then the canonical
// one (the sorted entry point's finish only orders it).
template <int NT, bool INDEX = false>
__device__ __forceinline__ void select_candidates(int ncand, uint32_t& prefix, int& shift, uint32_t& cnt,
                                                  uint32_t& need, uint32_t gt_base, uint32_t n,
                                                  uint32_t* sh_hist, const uint32_t* sh_ckey,
                                                  const int32_t* sh_cpos, int32_t* sh_raw, uint32_t* sh_scan,
                                                  uint32_t* sh_var, int tid, bool fill = false,
                                                  uint32_t* key_out = nullptr, bool canon = false) {
  while (shift > 0 && cnt != need) {
    for (int b = tid; b < kBinsNarrow; b += NT) sh_hist[b] = 0;
    __syncthreads();
    for (int i = tid; i < ncand; i += NT) {
      const uint32_t x = sh_ckey[i];
      if ((x >> shift) == prefix) atomicAdd(&sh_hist[(x >> (shift - 10)) & 1023u], 1u);
    }
    __syncthreads();
    find_threshold<NT, kBinsNarrow>(sh_hist, need, sh_scan, sh_var, tid);
    const uint32_t bin = uniform(sh_var[0]), gt = uniform(sh_var[1]);
    cnt = uniform(sh_var[2]);
    need -= gt;
    prefix = (prefix << 10) | bin;
    shift -= 10;
  }
  // With shift == 0 the keys left in the bin are identical: any `need` of
  // them, or with `canon` the `need` lowest positions.
  uint32_t vprefix = 0;
  int vshift = 32;
  if (canon && cnt != need) {
    lowest_positions<NT>(ncand, prefix, need, sh_ckey, sh_cpos, sh_hist, sh_scan, sh_var, tid, vprefix, vshift);
    cnt = need;
  }
  const uint32_t gt_end = n - need;
  if (tid == 0) {
    sh_var[8] = gt_base;
    sh_var[9] = 0;
  }
  if (fill)
    for (uint32_t j = (uint32_t)tid; j < n; j += NT) sh_raw[j] = -1;
  __syncthreads();
  for (int i = tid; i < ncand; i += NT) {
    const uint32_t key = sh_ckey[i];
    const uint32_t x = key >> shift;
    if (x > prefix) {
      const uint32_t s = atomicAdd(&sh_var[8], 1u);
      if (s < gt_end) {
        sh_raw[s] = INDEX ? i : sh_cpos[i];
        if (key_out) key_out[s] = key;
      }
    } else if (x == prefix && key != 0u && (vshift >= 32 || (~(uint32_t)sh_cpos[i] >> vshift) >= vprefix)) {
      const uint32_t e = atomicAdd(&sh_var[9], 1u);
      if (e < need) {
        sh_raw[gt_end + e] = INDEX ? i : sh_cpos[i];
        if (key_out) key_out[gt_end + e] = key;
      }
    }
  }
  __syncthreads();
}

// Raw loads of V float4 groups of a row chunk: group v of thread tid holds
// positions cbase + 4*tid + 4*NT*v + {0..3}.  One dwordx4 buffer load per group
// when the row is 16-byte aligned, else four dword loads.  The descriptor
// spans only the valid part of the chunk (whole 16-byte groups when aligned:
// the width is then a multiple of 4, so they stay inside the row), so the
// hardware returns 0 past seq_len and past the tensor without a branch.
// Nothing here consumes the data, so the loads stay in flight until the
// caller's first use (chunks are double-buffered this way).
// AUX is the loads' cache policy: kLoadStream (nt) for a row's first read,
// whose lines are not used again, kLoadReuse for the reads that revisit a
// row.  Measured on MI355X with this row-per-workgroup layout, nt loads read
// 537 MB at 6.9-7.1 TB/s against 6.1-6.3 TB/s for default-policy loads.
template <int NT, int V, int AUX = kLoadStream>
__device__ __forceinline__ void load_raw(uint32_t (&raw)[4 * V], const float* rowp, uint32_t cbase, uint32_t L,
                                         bool vec, int tid) {
  constexpr uint32_t span = (uint32_t)NT * 4u * V;
  const uint32_t rem = L > cbase ? L - cbase : 0u;
  const uint32_t nvalid = rem < span ? rem : span;
  const uint32_t nbytes = vec ? ((nvalid + 3u) & ~3u) * 4u : nvalid * 4u;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(rowp) + cbase, (short)0, (int)nbytes, kBufferWord3);
  const uint32_t voff = (uint32_t)tid * 16u;
  if (vec) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, v * (NT * 16), AUX);
#pragma unroll
      for (int i = 0; i < 4; ++i) raw[4 * v + i] = x[i];
    }
  } else {
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        raw[4 * v + i] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, voff, v * (NT * 16) + 4 * i, AUX);
  }
}

// Order key of raw slot j of a chunk at cbase, or 0 ("no element") past L.
template <int NT>
__device__ __forceinline__ uint32_t slot_key(uint32_t raw, int j, uint32_t cbase, uint32_t L, int tid) {
  // a scalar; L and cbase are below 2^31 (widths fit int32, cbase <= L + a chunk)
  const int32_t lim = (int32_t)L - (int32_t)cbase - (int32_t)((j >> 2) * NT * 4 + (j & 3));
  return (tid * 4 < lim) ? order_key_bits(raw) : 0u;
}

template <int NT, int V, int AUX = kLoadStream>
__device__ __forceinline__ void load_keys(uint32_t (&key)[4 * V], const float* rowp, uint32_t cbase, uint32_t L,
                                          bool vec, int tid) {
  load_raw<NT, V, AUX>(key, rowp, cbase, L, vec, tid);
#pragma unroll
  for (int j = 0; j < 4 * V; ++j) key[j] = slot_key<NT>(key[j], j, cbase, L, tid);
}

// SHORT (split kernel, rows cycled over slots): rows that fit one
// workgroup run in one workgroup of the slot (below).  A separate
// instantiation, so the one-pass split kernel keeps its split-only code.
template <int E, bool COOP, bool SHORT>
__device__ __forceinline__ void rows_body(KernelArgs a) {
  constexpr bool kOverlap = !SHORT;   // see the compaction below
  __shared__ uint32_t sh_hist[kBinsWide];
  __shared__ int32_t sh_raw[kMaxK + 64];   // + one trash word per lane
  __shared__ uint32_t sh_scan[64];   // block-scan wave totals, or the 64 coarse bins of find_threshold
  __shared__ uint32_t sh_var[16];
  __shared__ uint32_t sh_ckey[COOP ? kCandCap : 1];
  __shared__ int32_t sh_cpos[COOP ? kCandCap : 1];
  __shared__ int32_t sh_cout[COOP && kOverlap ? kCandCap : 1];   // the candidates' output values

  const int G = COOP ? a.wgs_per_row : 1;
  const int slot = (int)blockIdx.x / G;
  const int g = (int)blockIdx.x - slot * G;
  const int64_t C = (int64_t)kThreads * E;
  const int64_t W = a.width;
  const int k = a.k;
  uint32_t* fault = COOP ? a.ws + kHdrFault : nullptr;
  uint32_t* bar = COOP ? a.ws + kHdrWords + (size_t)slot * kBarWords : nullptr;
  uint32_t gen = (COOP && threadIdx.x == 0) ? g_load(bar + kBarGen) : 0u;   // see row_barrier
  uint32_t gave_up = 0;   // thread 0: a barrier wait of this workgroup gave up

  int nsplit = 0;   // split rows this slot has finished: picks the workspace region parity
  for (int it = 0;; ++it) {
    const int tid = opaque_tid();
    const int64_t row = (int64_t)slot + (int64_t)it * a.slots;
    if (row >= a.batch) break;
    // Without SHORT, a workgroup's share of the row does not depend on the
    // row's length, so its loads are issued before the length is read
    // (bounded by the width; the keys past the length are masked once it is
    // known) and the length's round trip overlaps them.
    const float* rowp = a.scores + row * W;
    const uint32_t c0 = COOP && !SHORT ? (uint32_t)g * (uint32_t)C : 0u;
    uint32_t key[E];
    if (!SHORT) load_raw<kThreads, E / 4>(key, rowp, c0, (uint32_t)W, a.vec != 0, tid);
    const int32_t sl = scalar_read(a.seq_lens, row);
    const int64_t L = sl < 0 ? 0 : ((int64_t)sl > W ? W : (int64_t)sl);
    const int n = L < (int64_t)k ? (int)L : k;
    // Rows that need no cross-workgroup merge -- every position selected
    // (L <= k), or, with SHORT, the row fits one workgroup's registers
    // (L <= C) -- run in one workgroup of the slot, the it-th row's in
    // workgroup it % G, so a run of them spreads over the slot; the slot's
    // other workgroups go on to its next row (whose first barrier, if it is
    // split, waits for this one).
    const int owner = SHORT ? it % G : 0;
    if (L <= (int64_t)k) {  // every valid position is selected (uniform over the row's workgroups)
      if (g == owner) write_row_output<kThreads>(a, row, L, n, true, sh_raw, tid);
      if (g == owner && tid == 0) record_selection(a, row, 0u, 32, (uint32_t)n, (uint32_t)n, 0u);
      continue;
    }
    const bool split = COOP && (!SHORT || L > C);   // the host launches the split kernel only with G > 1
    if (SHORT && !split && g != owner) continue;
    // Consecutive split rows of a slot alternate regions.  A region is reused
    // two split rows later, after every workgroup of the slot has passed the
    // in-between row's first barrier -- which the finisher that clears it
    // reaches only after clearing.
    uint32_t* region = split ? a.ws + kHdrWords + (size_t)a.ws_slots * kBarWords +
                                   ((size_t)slot * 2 + (size_t)(nsplit & 1)) * kRegionWords
                             : nullptr;
    nsplit += split ? 1 : 0;

    for (int j = tid; j < k; j += kThreads) sh_raw[j] = -1;

    // ---- this workgroup's share of the row in registers (one HBM read)
    if (SHORT) {
      const uint32_t cs = split ? (uint32_t)g * (uint32_t)C : 0u;
      load_keys<kThreads, E / 4>(key, rowp, cs, (uint32_t)L, a.vec != 0, tid);
    } else {
#pragma unroll
      for (int j = 0; j < E; ++j) key[j] = slot_key<kThreads>(key[j], j, c0, (uint32_t)L, tid);
    }
    const uint32_t pbase = (split ? (uint32_t)g * (uint32_t)C : 0u) + (uint32_t)tid * 4u;
    auto pos_of = [&](int j) -> int32_t {
      return (int32_t)(pbase + (uint32_t)(j >> 2) * (kThreads * 4) + (uint32_t)(j & 3));
    };

    // ---- radix passes: 12, 10, 10 bits, MSB first
    uint32_t prefix = 0, need = (uint32_t)n, cnt = 0;
    int shift = 32, mode = kModeNone, pass = 0;
    for (pass = 0; pass < 3; ++pass) {
      const int nb = pass == 0 ? kBinsWide : kBinsNarrow;
      for (int b = tid; b < nb; b += kThreads) sh_hist[b] = 0;
      __syncthreads();
      launder(key);
      // Pass 0 of a split row pushes only bins >= t_s: the row has at least
      // `need` keys at or above t_s, so its threshold bin is >= t_s, and
      // every bin the merged search can reach is complete.
      uint32_t push_from = 0;
      if (pass == 0) push_from = hist_pass0<E>(key, need, sh_hist, sh_scan, sh_var, tid, split);
      else hist_resident<E>(key, pass, prefix, sh_hist);
      __syncthreads();
      if (split) {
        uint32_t* gh = region + (pass == 0 ? kRegHist0 : pass == 1 ? kRegHist1 : kRegHist2);
        for (int b = tid; b < nb; b += kThreads) {
          const uint32_t c = sh_hist[b];
          if (c && (uint32_t)b >= push_from) g_add(gh + b, c);
        }
        row_barrier(bar, G, g, gen, fault, a.spin_limit, gave_up, tid);
        for (int b = tid; b < nb; b += kThreads) sh_hist[b] = g_load(gh + b);
        __syncthreads();
      }
      if (pass == 0) find_threshold<kThreads, kBinsWide>(sh_hist, need, sh_scan, sh_var, tid);
      else find_threshold<kThreads, kBinsNarrow>(sh_hist, need, sh_scan, sh_var, tid);
      const uint32_t bin = uniform(sh_var[0]), gt = uniform(sh_var[1]);
      cnt = uniform(sh_var[2]);
      need -= gt;
      prefix = pass == 0 ? bin : ((prefix << 10) | bin);
      shift = pass == 0 ? 20 : shift - 10;
      if (cnt == need) {
        mode = kModeTakeAll;
        break;
      }
      if (pass == 2) {
        mode = kModeTies;
        break;
      }
      if (split && cnt <= (uint32_t)kCandCap) {
        mode = kModeCands;
        break;
      }
    }

    // ---- compaction: strictly-greater keys take slots [0, n - need); keys in
    // the threshold bin take the tie slots [n - need, n) or become candidates.
    const uint32_t n_gt = (uint32_t)n - need;
    launder(key);
    uint32_t cg = 0, ce = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const uint32_t x = key[j];
      const uint32_t xp = x >> shift;
      cg += xp > prefix ? 1u : 0u;
      ce += (xp == prefix && x != 0u) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t off = block_exclusive_scan<kThreads>((cg << 17) | ce, sh_scan, tot, tid);
    uint32_t off_g = off >> 17, off_e = off & 0x1FFFFu;
    // One-pass split rows (kOverlap) take their offsets while the selected
    // keys are staged and gathered, and hand the finisher candidates with
    // their output values.  Rows cycled over slots keep the staged-slot
    // form (offsets first, then the gathers), measured faster there: the
    // cycled batch's finish overlaps the slot's next row, and the overlapped
    // form took it from 48.1 to 49.4 us.
    if constexpr (kOverlap) {
      // Split rows: the workgroup's slots come from one atomic on the row's
      // counter (the strictly-greater count in the high word, the threshold-bin
      // count in the low word; a row's total is below 2^31, so it never
      // carries).  While it is in flight, the selected keys are staged in LDS
      // at their ranks within the workgroup and the page-table entry of every
      // staged key is gathered: the outputs (and the candidates' output values)
      // are stored as soon as the offsets arrive, with no gather after them.
      const uint32_t tg = tot >> 17, te = tot & 0x1FFFFu;
      uint64_t base = 0;
      if (split && tid == 0)
        base = g_add64_ret(reinterpret_cast<uint64_t*>(region + kRegCtr + kCtrSlots), ((uint64_t)tg << 32) | (uint64_t)te);
      // Selected keys are rare: a wave skips a register slot unless one of its
      // lanes holds a key at or above the threshold prefix.  Inside, lanes that
      // have nothing to store write a private trash word instead of branching.
      // Split rows stage greater keys at ranks [0, tg) of sh_raw (tg <= n -
      // need <= kMaxK) and threshold-bin keys at ranks [0, min(te, kCandCap))
      // of sh_ckey / sh_cpos (a rank past that can be neither a candidate nor
      // a tie slot).
      const uint32_t trash = (uint32_t)kMaxK + (uint32_t)(tid & 63);
      launder(key);   // recompute the compares here instead of keeping 2E masks from the counting loop
  #pragma unroll
      for (int j = 0; j < E; ++j) {
        const uint32_t x = key[j];
        const uint32_t xp = x >> shift;
        const bool isg = xp > prefix;
        const bool ise = (xp == prefix) && (x != 0u);
        if (__ballot(isg || ise) == 0ull) continue;
        const uint32_t sg = off_g, se = off_e;
        off_g += isg ? 1u : 0u;
        off_e += ise ? 1u : 0u;
        if (!split) {
          const uint32_t slot = (isg && sg < n_gt) ? sg : ((ise && se < need) ? n_gt + se : trash);
          sh_raw[slot] = pos_of(j);
        } else {
          if (isg) sh_raw[sg] = pos_of(j);
          if (ise && se < (uint32_t)kCandCap) {
            sh_ckey[se] = x;
            sh_cpos[se] = pos_of(j);
          }
        }
      }
      if (split) {
        __syncthreads();
        const uint32_t te_staged = te < (uint32_t)kCandCap ? te : (uint32_t)kCandCap;
        const int ps = a.log2_page;
        const uint32_t pmask = (1u << ps) - 1u;
        const int32_t* pt = a.page_table + row * a.pages_per_row;
        auto transformed = [&](int32_t r, int32_t page) -> int32_t {
          return (int64_t)(r >> ps) < a.pages_per_row ? (int32_t)(((uint32_t)page << ps) | ((uint32_t)r & pmask)) : -1;
        };
        // The page values go to LDS (the histogram and the finisher's output
        // list are free now), so nothing is held in registers across the wait:
        // greater keys' pages at sh_hist[i], threshold-bin keys' at sh_cout[i].
        int32_t* const g_page = reinterpret_cast<int32_t*>(sh_hist);
        for (uint32_t i = (uint32_t)tid; i < tg; i += kThreads) {
          const int32_t r = sh_raw[i];
          g_page[i] = (int64_t)(r >> ps) < a.pages_per_row ? pt[r >> ps] : 0;
        }
        for (uint32_t i = (uint32_t)tid; i < te_staged; i += kThreads) {
          const int32_t r = sh_cpos[i];
          sh_cout[i] = (int64_t)(r >> ps) < a.pages_per_row ? pt[r >> ps] : 0;
        }
        if (tid == 0) {
          sh_var[4] = (uint32_t)(base >> 32);
          sh_var[5] = (uint32_t)base;
        }
        __syncthreads();
        const uint32_t base_g = uniform(sh_var[4]), base_e = uniform(sh_var[5]);
        int32_t* o = a.out + row * (int64_t)k;
        int32_t* orw = a.out_raw ? a.out_raw + row * (int64_t)k : nullptr;
        for (uint32_t i = (uint32_t)tid; i < tg; i += kThreads) {
          const uint32_t slot = base_g + i;
          if (slot < n_gt) {
            const int32_t r = sh_raw[i];
            o[slot] = transformed(r, g_page[i]);
            if (orw) orw[slot] = r;
          }
        }
        for (uint32_t i = (uint32_t)tid; i < te_staged; i += kThreads) {
          const uint32_t e = base_e + i;
          const int32_t r = sh_cpos[i];
          if (mode == kModeCands) {
            if (e < (uint32_t)kCandCap) {
              const uint32_t x = sh_ckey[i];
              g_store(region + kRegCandKey + e, x);
              g_store(region + kRegCandPos + e, (uint32_t)r);
              g_store(region + kRegCandOut + e, (uint32_t)transformed(r, sh_cout[i]));
              // the candidates' next digit, merged in the next pass's
              // histogram (unused in this mode, zero at rest): the finisher
              // starts from it instead of histogramming the candidates
              g_add(region + (shift == 20 ? kRegHist1 : kRegHist2) + ((x >> (shift - 10)) & 1023u), 1u);
            }
          } else if (e < need) {
            o[n_gt + e] = transformed(r, sh_cout[i]);
            if (orw) orw[n_gt + e] = r;
          }
        }
      }
    } else {
      if (split) {
        if (tid == 0) {
          // both offsets from one atomic (one round trip instead of two): the
          // strictly-greater count in the high word, the threshold-bin count in
          // the low word (a row's total is below 2^31, so it never carries)
          const uint32_t tg = tot >> 17, te = tot & 0x1FFFFu;
          const uint64_t old = g_add64_ret(reinterpret_cast<uint64_t*>(region + kRegCtr + kCtrSlots),
                                           ((uint64_t)tg << 32) | (uint64_t)te);
          sh_var[4] = (uint32_t)(old >> 32);
          sh_var[5] = (uint32_t)old;
          sh_var[7] = 0u;   // this workgroup's (slot, position) pairs staged below
        }
        __syncthreads();
        off_g += uniform(sh_var[4]);
        off_e += uniform(sh_var[5]);
      }
      // Selected keys are rare: a wave skips a register slot unless one of its
      // lanes holds a key at or above the threshold prefix.  Inside, lanes that
      // have nothing to store write a private trash word instead of branching.
      const uint32_t trash = (uint32_t)kMaxK + (uint32_t)(tid & 63);
      // Split rows stage each final (slot, position) pair in LDS (sh_ckey /
      // sh_raw; a row has n <= kMaxK slots, so fewer pairs than either holds)
      // and write them after the loop: a page-table gather per selected key
      // inside the loop would make each register slot wait out a load.
      auto stage_slot = [&](uint32_t slot, int32_t pos) {
        const uint32_t li = atomicAdd(&sh_var[7], 1u);
        sh_ckey[li] = slot;
        sh_raw[li] = pos;
      };
      launder(key);   // recompute the compares here instead of keeping 2E masks from the counting loop
  #pragma unroll
      for (int j = 0; j < E; ++j) {
        const uint32_t x = key[j];
        const uint32_t xp = x >> shift;
        const bool isg = xp > prefix;
        const bool ise = (xp == prefix) && (x != 0u);
        if (__ballot(isg || ise) == 0ull) continue;
        const uint32_t sg = off_g, se = off_e;
        off_g += isg ? 1u : 0u;
        off_e += ise ? 1u : 0u;
        if (!split) {
          const uint32_t slot = (isg && sg < n_gt) ? sg : ((ise && se < need) ? n_gt + se : trash);
          sh_raw[slot] = pos_of(j);
        } else if (mode == kModeCands) {
          if (isg && sg < n_gt) stage_slot(sg, pos_of(j));
          if (ise && se < (uint32_t)kCandCap) {
            g_store(region + kRegCandKey + se, x);
            g_store(region + kRegCandPos + se, (uint32_t)pos_of(j));
          }
        } else {
          const uint32_t slot = (isg && sg < n_gt) ? sg : ((ise && se < need) ? n_gt + se : 0xFFFFFFFFu);
          if (slot != 0xFFFFFFFFu) stage_slot(slot, pos_of(j));
        }
      }
      if (split) {
        // The staged slots are final: write them through the page table, every
        // gather in flight at once.
        __syncthreads();
        const uint32_t nsel = uniform(sh_var[7]);
        for (uint32_t i = (uint32_t)tid; i < nsel; i += kThreads) write_slot(a, row, sh_ckey[i], sh_raw[i]);
      }
    }
    if (!split) {
      __syncthreads();
      write_row_output<kThreads>(a, row, L, n, false, sh_raw, tid);
      if (tid == 0) record_selection(a, row, prefix, shift, need, cnt, 1u);
      continue;
    }

    // ---- the last workgroup to leave the row finishes it
    wave_mem_drain();
    __syncthreads();
    if (tid == 0) {
      const uint32_t old = g_add_ret(region + kRegCtr + kCtrExit, 1u);
      wave_mem_drain();
      sh_var[6] = (old == (uint32_t)G - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (!uniform(sh_var[6])) continue;

    // A split row has L > k, so n = k: every slot below n_gt (all n of them
    // outside the candidates mode) was written by the workgroup whose key
    // took it; the candidates fill [n_gt, n).
    if constexpr (kOverlap) {
      if (mode == kModeCands) {
        // Each candidate arrives with its output value (its workgroup did the
        // page-table gather): the selected ones are written with no gather.
        // The candidates' next digit arrives merged (the workgroups counted
        // it), so the first refinement needs no pass over them.
        const int ncand = (int)(cnt < (uint32_t)kCandCap ? cnt : (uint32_t)kCandCap);
        static_assert(kThreads == kBinsNarrow, "one merged next-digit bin per thread");
        const uint32_t sub = g_load(region + (shift == 20 ? kRegHist1 : kRegHist2) + tid);
        // every candidate load in flight before the first is stored
        constexpr int kPer = kCandCap / kThreads;
        uint32_t ck[kPer], cp[kPer], co[kPer];
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
          const int i = tid + q * kThreads;
          if (i < ncand) {
            ck[q] = g_load(region + kRegCandKey + i);
            cp[q] = g_load(region + kRegCandPos + i);
            co[q] = g_load(region + kRegCandOut + i);
          }
        }
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
          const int i = tid + q * kThreads;
          if (i < ncand) {
            sh_ckey[i] = ck[q];
            sh_cpos[i] = (int32_t)cp[q];
            sh_cout[i] = (int32_t)co[q];
          }
        }
        sh_hist[tid] = sub;
        __syncthreads();
        find_threshold<kThreads, kBinsNarrow>(sh_hist, need, sh_scan, sh_var, tid);
        {
          const uint32_t bin = uniform(sh_var[0]), gt = uniform(sh_var[1]);
          cnt = uniform(sh_var[2]);
          need -= gt;
          prefix = (prefix << 10) | bin;
          shift -= 10;
        }
        select_candidates<kThreads, true>(ncand, prefix, shift, cnt, need, n_gt, (uint32_t)n, sh_hist, sh_ckey, sh_cpos,
                                          sh_raw, sh_scan, sh_var, tid);
        __syncthreads();
        // A split row has L > k: n = k, and the candidates fill [n_gt, k).
        int32_t* o = a.out + row * (int64_t)k;
        int32_t* orw = a.out_raw ? a.out_raw + row * (int64_t)k : nullptr;
        for (int j = (int)n_gt + tid; j < k; j += kThreads) {
          const int i = sh_raw[j];
          const bool ok = i >= 0 && i < ncand;
          o[j] = ok ? sh_cout[i] : -1;
          if (orw) orw[j] = ok ? sh_cpos[i] : -1;
        }
      }
    } else {
      if (mode == kModeCands) {
        const int ncand = (int)(cnt < (uint32_t)kCandCap ? cnt : (uint32_t)kCandCap);
        for (int i = tid; i < ncand; i += kThreads) {
          sh_ckey[i] = g_load(region + kRegCandKey + i);
          sh_cpos[i] = (int32_t)g_load(region + kRegCandPos + i);
        }
        __syncthreads();
        select_candidates<kThreads>(ncand, prefix, shift, cnt, need, n_gt, (uint32_t)n, sh_hist, sh_ckey, sh_cpos, sh_raw,
                          sh_scan, sh_var, tid);
        __syncthreads();
        write_row_output<kThreads>(a, row, L, n, false, sh_raw, tid, nullptr, (int)n_gt);
      }
    }
    if (tid == 0) record_selection(a, row, prefix, shift, need, cnt, 1u);
    // leave the region zeroed for the row this slot handles two iterations on
    for (int b = tid; b < kBinsWide; b += kThreads) g_store(region + kRegHist0 + b, 0u);
    for (int b = tid; b < kBinsNarrow; b += kThreads) {
      g_store(region + kRegHist1 + b, 0u);
      g_store(region + kRegHist2 + b, 0u);
    }
    if (tid < 64) g_store(region + kRegCtr + tid, 0u);
    __syncthreads();
  }
  if (COOP) launch_exit(a, gave_up, &sh_var[15], opaque_tid());
}

template <int E, bool COOP, bool SHORT>
__global__ void __launch_bounds__(kThreads) rows_kernel(KernelArgs a) {
  rows_body<E, COOP, SHORT>(a);
}

// Cycled split rows in one of two shapes, E = 64 (a's wgs_per_row and slots)
// or E = 16 (g16 and slots16), both in one launch whose grid holds the larger
// of their grids.  Every workgroup counts the rows longer than a.choice_len
// (the same count everywhere), and the launch takes the E = 16 shape if there
// are at most a.choice_rows of them.  Workgroups past the taken shape's grid
// only check in at the launch's exit count.
__global__ void __launch_bounds__(kThreads) rows_pair_kernel(KernelArgs a, int32_t g16, int32_t slots16) {
  __shared__ uint32_t sh_long;
  const int t0 = opaque_tid();
  if (t0 == 0) sh_long = 0u;
  __syncthreads();
  uint32_t c = 0;
  for (int r = t0; r < a.batch; r += kThreads)   // min(len, W) > choice_len
    c += (a.width > (int64_t)a.choice_len && a.seq_lens[r] > a.choice_len) ? 1u : 0u;
  if (c != 0u) atomicAdd(&sh_long, c);
  __syncthreads();
  const bool few = uniform(sh_long) <= (uint32_t)a.choice_rows;
  const int64_t grid = few ? (int64_t)slots16 * g16 : (int64_t)a.slots * a.wgs_per_row;
  if ((int64_t)blockIdx.x >= grid) {
    launch_exit(a, 0u, &sh_long, opaque_tid());
    return;
  }
  if (few) {
    KernelArgs b = a;
    b.wgs_per_row = g16;
    b.slots = slots16;
    rows_body<16, true, true>(b);
  } else {
    rows_body<64, true, true>(a);
  }
}

// ---------------------------------------------------------------------------
// Helpers of the streaming kernel (stream_rows_kernel, below).
// ---------------------------------------------------------------------------

// Stream-kernel LDS words (sh_var indices).
enum : int { kVarCandCount = 10, kVarOverflow = 11, kVarGt = 12, kVarEq = 13, kVarAbove = 14 };

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// How gated_append tests a raw score against the gate key.
enum : int {
  kGatePositive = 0,   // every slot valid, gate >= key(+0): raw bits compare as signed ints
  kGateAny = 1,        // every slot valid
  kGateChecked = 2,    // slots past L are absent
};

// Appends the keys >= gate (gate >= 1, so key 0 never passes) of one chunk
// of raw scores to the candidate list: slots come from one LDS atomic per
// wave, each passing lane's slot from its rank in the wave's ballot.  Slots
// past CAP land in the trash entry CAP (the count still grows: overflow).
// With kGatePositive the test is one signed compare: a float at or above a
// non-negative gate has a non-negative bit pattern, ordered like its key, and
// every negative float (sign bit set) is a negative int.
template <int NT, int CAP, int N, int FORM>
__device__ __forceinline__ void gated_append(const uint32_t (&raw)[N], uint32_t cbase, uint32_t L, uint32_t gate,
                                             uint32_t* sh_ckey, int32_t* sh_cpos, uint32_t* sh_var, int tid) {
  const int32_t graw = (int32_t)(gate ^ 0x80000000u);
  uint64_t m[N];
  uint32_t tot = 0;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    bool pass;
    if (FORM == kGatePositive) pass = (int32_t)raw[j] >= graw;
    else if (FORM == kGateAny) pass = order_key_bits(raw[j]) >= gate;
    else pass = slot_key<NT>(raw[j], j, cbase, L, tid) >= gate;
    m[j] = __ballot(pass);
    tot += (uint32_t)__popcll(m[j]);
  }
  if (tot == 0u) return;
  uint32_t base = 0;
  if ((tid & 63) == 0) base = atomicAdd(&sh_var[kVarCandCount], tot);
  base = __builtin_amdgcn_readfirstlane(base);
  const uint32_t p0 = cbase + (uint32_t)tid * 4u;
  const int lane = tid & 63;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    if (m[j] == 0ull) continue;
    if ((m[j] >> lane) & 1ull) {
      uint32_t slot = base + lanes_below(m[j]);
      slot = slot < (uint32_t)CAP ? slot : (uint32_t)CAP;
      sh_ckey[slot] = order_key_bits(raw[j]);
      sh_cpos[slot] = (int32_t)(p0 + (uint32_t)(j >> 2) * (NT * 4) + (uint32_t)(j & 3));
    }
    base += (uint32_t)__popcll(m[j]);
  }
}

// 12-bit-bin histogram of the first `ncand` candidates' keys (cleared first).
template <int NT>
__device__ __forceinline__ void list_histogram(uint32_t ncand, const uint32_t* sh_ckey, uint32_t* sh_hist, int tid) {
  for (int b = tid; b < kBinsWide; b += NT) sh_hist[b] = 0u;
  __syncthreads();
  for (uint32_t i = (uint32_t)tid; i < ncand; i += NT) atomicAdd(&sh_hist[sh_ckey[i] >> 20], 1u);
  __syncthreads();
}

// Raises the gate to the lowest key of the threshold bin of the listed keys
// (every key >= gate seen so far, unless the list has overflowed; a subset
// still gives a bin that at least n keys of the row reach) and drops the
// candidates below it.  Uniform; returns the new gate.  The list is compacted in place in rounds of 2 * NT entries: a
// round's entries are read into registers before any is written, and kept
// entries only move down (to positions below the round's end), so no unread
// entry is overwritten.
template <int NT, int CAP>
__device__ __forceinline__ uint32_t raise_gate(uint32_t gate, uint32_t n, uint32_t* sh_hist, uint32_t* sh_ckey,
                                               int32_t* sh_cpos, uint32_t* sh_scan, uint32_t* sh_var, int tid) {
  const uint32_t count = uniform(sh_var[kVarCandCount]);
  const uint32_t ncur = count < (uint32_t)CAP ? count : (uint32_t)CAP;
  list_histogram<NT>(ncur, sh_ckey, sh_hist, tid);
  find_threshold<NT, kBinsWide>(sh_hist, n, sh_scan, sh_var, tid);
  const uint32_t t = uniform(sh_var[0]);
  if (t <= (gate >> 20)) return gate;
  uint32_t kept = 0;   // uniform: entries kept by earlier rounds
  for (uint32_t r0 = 0; r0 < ncur; r0 += 2u * NT) {
    const uint32_t i0 = r0 + (uint32_t)tid * 2u;
    const uint32_t k0 = i0 < ncur ? sh_ckey[i0] : 0u, k1 = i0 + 1u < ncur ? sh_ckey[i0 + 1u] : 0u;
    const int32_t p0 = i0 < ncur ? sh_cpos[i0] : 0, p1 = i0 + 1u < ncur ? sh_cpos[i0 + 1u] : 0;
    const bool q0 = (k0 >> 20) >= t, q1 = (k1 >> 20) >= t;
    uint32_t total;
    uint32_t off = kept + block_exclusive_scan<NT>((q0 ? 1u : 0u) + (q1 ? 1u : 0u), sh_scan, total, tid);
    if (q0) {
      sh_ckey[off] = k0;
      sh_cpos[off] = p0;
      ++off;
    }
    if (q1) {
      sh_ckey[off] = k1;
      sh_cpos[off] = p1;
    }
    kept += total;
    __syncthreads();
  }
  if (tid == 0) {
    if (count > (uint32_t)CAP) sh_var[kVarOverflow] = 1u;   // keys were lost: redo the row
    sh_var[kVarCandCount] = kept;
  }
  __syncthreads();
  return t << 20;
}

// One pass over the row from memory, for the overflow path.  Keys below
// `floor` (>= 1) are treated as absent: when at least n keys lie at or above
// the streaming gate, the gate is the floor and every count stays consistent
// with the histogram, which holds only keys >= gate in the gate's own bin.
// With mode 3, histograms every key's 12-bit bin; with mode 0, histograms the
// next 10-bit digit of the keys whose key >> shift equals prefix; with mode 1,
// writes keys above the bin to slots [0, n - need) and collects the bin's keys
// as candidates; with mode 2 (final digit, or the whole bin is selected),
// writes keys above the bin to [0, n - need) and `need` keys of the bin to
// [n - need, n).
template <int NT, int CAP, int CV>
__device__ __forceinline__ void restream_pass(int mode, const float* rowp, uint32_t L, bool vec, uint32_t floor,
                                              uint32_t prefix, int shift, uint32_t need, uint32_t n, uint32_t* sh_hist,
                                              uint32_t* sh_ckey, int32_t* sh_cpos, int32_t* sh_raw,
                                              uint32_t* sh_var, int tid) {
  constexpr uint32_t span = (uint32_t)NT * 4u * CV;
  const uint32_t gt_end = n - need;
  for (uint32_t c = 0; c < L; c += span) {
    uint32_t key[4 * CV];
    load_keys<NT, CV, kLoadReuse>(key, rowp, c, L, vec, tid);
    const uint32_t p0 = c + (uint32_t)tid * 4u;
#pragma unroll
    for (int j = 0; j < 4 * CV; ++j) {
      const uint32_t x = key[j];
      if (x < floor) continue;
      if (mode == 3) {
        atomicAdd(&sh_hist[x >> 20], 1u);
        continue;
      }
      const uint32_t xp = x >> shift;
      const int32_t pos = (int32_t)(p0 + (uint32_t)(j >> 2) * (NT * 4) + (uint32_t)(j & 3));
      if (mode == 0) {
        if (xp == prefix) atomicAdd(&sh_hist[(x >> (shift - 10)) & 1023u], 1u);
      } else if (xp > prefix) {
        const uint32_t s = atomicAdd(&sh_var[kVarGt], 1u);
        if (s < gt_end) sh_raw[s] = pos;
      } else if (xp == prefix) {
        const uint32_t e = atomicAdd(&sh_var[kVarEq], 1u);
        if (mode == 1) {
          if (e < (uint32_t)CAP) {
            sh_ckey[e] = x;
            sh_cpos[e] = pos;
          }
        } else if (e < need) {
          sh_raw[gt_end + e] = pos;
        }
      }
    }
  }
  __syncthreads();
}

// Wave priority for a queued row: the rank of its ticket within its round of
// `grid` tickets, in quarters (0 = among the first to finish a row).
__device__ __forceinline__ void set_row_priority(uint32_t row, uint32_t grid) {
  const uint32_t q = ((row % grid) * 4u) / grid;
  if (q == 0u) __builtin_amdgcn_s_setprio(0);
  else if (q == 1u) __builtin_amdgcn_s_setprio(1);
  else if (q == 2u) __builtin_amdgcn_s_setprio(2);
  else __builtin_amdgcn_s_setprio(3);
}

// Sample rank the streaming gate is set at.  The first S of a row's L
// positions hold on average mu = n*S/L of the row's n largest keys (a
// hypergeometric count); the gate sits at the m-th largest sampled key with
// m = mu + 7 sqrt(mu) + 6 (at most n).  When the row's large keys are spread
// along it, fewer than n of its keys lie at or above the gate with
// probability below 1e-11 for every row shape up to 1M positions and k 2048;
// such a row is detected at the end and finished exactly from memory (one
// workgroup re-reads it, so a rare one still costs the whole launch tens of
// microseconds).  m = n, a gate that holds for any row, when the sample is
// the row.
__device__ __forceinline__ uint32_t gate_rank(uint32_t n, uint32_t S, uint32_t L) {
  const float mu = (float)n * (float)S / (float)L;
  const float m = mu + 7.0f * sqrtf(mu) + 6.0f;
  return m < (float)n ? (uint32_t)m : n;
}

// ---------------------------------------------------------------------------
// Streaming one-workgroup-per-row kernel (large batches).
//
// Holding a 64K row in registers leaves one row per CU and nothing to overlap
// its radix passes with; streaming keeps several rows in flight per CU.
//   1. Sample: the first NT*4*SV positions are histogrammed in full; the
//      sample's threshold bin is a gate such that at least n keys of the row
//      lie at or above it.
//   2. Stream: every key at or above the gate is counted (so the histogram is
//      exact for every bin >= gate) and appended to an LDS candidate list;
//      slots come from wave ballots, one LDS atomic per wave per chunk.  When
//      the list fills, the gate is raised to the threshold bin of the keys
//      seen so far (still a valid lower bound) and the list is compacted.
//   3. The threshold bin comes from the exact histogram; the remaining digits
//      run on the candidates only.
// If the list overflows anyway (adversarial rows: a single bin holding more
// keys than the list), the row is redone by re-streaming it from memory with
// one more digit per pass until the threshold bin fits (exact, slower).
//
// Rows beyond the first grid come from a queue (a ticket counter in the
// workspace header) rather than a fixed stride: workgroups that share a CU
// are not served memory equally (older waves win), so a fixed two rows each
// leaves the youngest finishing tens of microseconds after the oldest.  The
// ticket is taken once a row's streaming ends; the last workgroup to run out
// of rows puts the counters back to zero for the next launch.  A ticket's
// rank within its round of `grid` tickets says how many workgroups finished a
// row before this one; the later it came, the higher the wave priority the
// workgroup runs its next row at, which offsets the age order of the memory
// arbitration and evens out the finishing times.
//
//
// NT threads per workgroup, SV / CV float4 groups per thread in the sample /
// in each streamed chunk, NBUF chunks in flight (a register ring), CAP
// candidates in LDS, WAVES = waves per SIMD the register budget is set for.
// With PTL, a row's page table (up to 4 NT entries) is requested before the
// row is finished and staged in LDS for the output pass, taking the gather's
// dependent global loads off the row's critical path.
// ---------------------------------------------------------------------------
template <int NT, int SV, int CV, int NBUF, int CAP, int WAVES, bool PTL, bool VEC>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(WAVES, WAVES)))
stream_rows_kernel(KernelArgs a) {
  constexpr uint32_t kSampleSpan = (uint32_t)NT * 4u * SV;
  constexpr uint32_t kChunkSpan = (uint32_t)NT * 4u * CV;
  constexpr uint32_t kRefresh = CAP - CAP / 4;   // raise the gate once the list is this full
  static_assert(CAP >= kBinsNarrow, "the candidate list doubles as the gate's sub-histogram");
  __shared__ uint32_t sh_hist[kBinsWide];
  __shared__ uint32_t sh_ckey[CAP + 1];   // + the trash entry of an overflowing list
  __shared__ int32_t sh_cpos[CAP + 1];
  __shared__ uint32_t sh_scan[64];   // the 64 coarse bins of find_threshold
  // The selected positions share the histogram's upper half: once the row's
  // 12-bit threshold bin is known, only 10-bit digits (bins [0, 1024)) are
  // histogrammed until the row is written.
  static_assert(kBinsWide - kMaxK >= kBinsNarrow, "selected positions alias the histogram's upper half");
  int32_t* const sh_raw = reinterpret_cast<int32_t*>(sh_hist + (kBinsWide - kMaxK));
  __shared__ uint32_t sh_var[16];
  __shared__ uint32_t sh_next_row;
  __shared__ int32_t sh_next_len;   // seq_lens[next row], loaded while this row finishes

  const int64_t W = a.width;
  const int k = a.k;
  constexpr bool vec = VEC;   // a compile-time load form: see the ring below
  // The host passes a workspace only when there are more rows than workgroups.
  uint32_t* const queue = a.ws != nullptr ? a.ws + kHdrRowTicket : nullptr;
  const uint32_t grid = gridDim.x;
  uint32_t row = blockIdx.x;
  int32_t seq = row < (uint32_t)a.batch ? (int32_t)uniform((uint32_t)a.seq_lens[row]) : 0;
  while (row < (uint32_t)a.batch) {
    const int tid = opaque_tid();
    const int64_t L64 = seq < 0 ? 0 : ((int64_t)seq > W ? W : (int64_t)seq);
    const uint32_t L = (uint32_t)L64;
    const int n = L64 < (int64_t)k ? (int)L64 : k;
    if (L64 <= (int64_t)k) {
      __syncthreads();   // every wave has read the previous row's ticket
      if (tid == 0) {
        const uint32_t nx = queue != nullptr ? grid + take_ticket(queue) : row + grid;
        sh_next_row = nx;
        sh_next_len = nx < (uint32_t)a.batch ? a.seq_lens[nx] : 0;
        record_selection(a, row, 0u, 32, (uint32_t)n, (uint32_t)n, 0u);
      }
      write_row_output<NT>(a, row, L64, n, true, sh_raw, tid);
      __syncthreads();
      row = uniform(sh_next_row);
      seq = (int32_t)uniform((uint32_t)sh_next_len);
      continue;
    }
    for (int b = tid; b < kBinsWide; b += NT) sh_hist[b] = 0;
    if (tid < 16) sh_var[tid] = 0;
    const float* rowp = a.scores + row * W;
    __syncthreads();

    // 1. sample: full histogram of the first kSampleSpan positions (the
    // first NBUF streamed chunks' loads are issued before the sample is used)
    //
    // The ring's loads are issued unconditionally, also for chunks past the
    // row (their descriptor covers nothing: no memory is read, they return
    // zeros), and the load form is fixed at compile time.  Then every path
    // issues the same loads in the same order, and the compiler's per-use
    // waits can leave the later chunks in flight.  A branch around a load,
    // or a vec / scalar choice made at run time, gives it a path with fewer
    // loads outstanding, and its waits then hold each chunk's use until the
    // chunks requested after it have arrived as well.
    uint32_t sk[4 * SV];   // the sample's raw scores
    load_raw<NT, SV>(sk, rowp, 0u, L, vec, tid);
    const uint32_t nch = L > kSampleSpan ? (L - kSampleSpan + kChunkSpan - 1) / kChunkSpan : 0u;
    uint32_t ring[NBUF][4 * CV];
#pragma unroll
    for (int b = 0; b < NBUF; ++b) load_raw<NT, CV>(ring[b], rowp, kSampleSpan + (uint32_t)b * kChunkSpan, L, vec, tid);
#pragma unroll
    for (int j = 0; j < 4 * SV; ++j) {
      const uint32_t x = slot_key<NT>(sk[j], j, 0u, L, tid);
      if (x) atomicAdd(&sh_hist[x >> 20], 1u);
    }
    __syncthreads();
    const uint32_t m = gate_rank((uint32_t)n, L < kSampleSpan ? L : kSampleSpan, L);
    find_threshold<NT, kBinsWide>(sh_hist, m, sh_scan, sh_var, tid);
    // The gate is refined inside the sample's bin with the next 10 key bits,
    // so that about m/S of the streamed keys pass it rather than a whole
    // bin's worth more.  The (still empty) candidate list holds the
    // sub-histogram meanwhile.
    const uint32_t gbin = uniform(sh_var[0]), gneed = m - uniform(sh_var[1]);
    for (int b = tid; b < kBinsNarrow; b += NT) sh_ckey[b] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4 * SV; ++j) {
      const uint32_t x = slot_key<NT>(sk[j], j, 0u, L, tid);
      if (x != 0u && (x >> 20) == gbin) atomicAdd(&sh_ckey[(x >> 10) & 1023u], 1u);
    }
    __syncthreads();
    find_threshold<NT, kBinsNarrow>(sh_ckey, gneed, sh_scan, sh_var, tid);
    uint32_t gate = (gbin << 20) | (uniform(sh_var[0]) << 10);
    if (gate == 0u) gate = 1u;
    {   // in two halves: fewer ballot masks live at once (register pressure)
      static_assert(SV % 2 == 0, "the sample is appended in two halves");
      uint32_t lo[2 * SV], hi[2 * SV];
#pragma unroll
      for (int j = 0; j < 2 * SV; ++j) {
        lo[j] = sk[j];
        hi[j] = sk[2 * SV + j];
      }
      constexpr uint32_t half = (uint32_t)NT * 4u * (SV / 2);
      gated_append<NT, CAP, 2 * SV, kGateChecked>(lo, 0u, L, gate, sh_ckey, sh_cpos, sh_var, tid);
      gated_append<NT, CAP, 2 * SV, kGateChecked>(hi, half, L, gate, sh_ckey, sh_cpos, sh_var, tid);
    }

    // 2. stream the rest through the ring: chunk i + NBUF is requested as soon
    // as chunk i's registers are consumed
    // next row's ticket, taken at the start of the last ring cycle (its return
    // is first needed when the stream ends)
    uint32_t next = row + grid;
    const uint32_t last_cycle = nch > 0u ? ((nch - 1u) / NBUF) * NBUF : 0u;
    if (queue != nullptr && tid == 0 && nch == 0u) next = grid + take_ticket(queue);
    for (uint32_t i = 0; i < nch; i += NBUF) {
      if (queue != nullptr && tid == 0 && i == last_cycle) next = grid + take_ticket(queue);
#pragma unroll
      for (int b = 0; b < NBUF; ++b) {
        const uint32_t idx = i + (uint32_t)b;
        if (idx < nch) {
          const uint32_t cbase = kSampleSpan + idx * kChunkSpan;
          if (cbase + kChunkSpan > L)
            gated_append<NT, CAP, 4 * CV, kGateChecked>(ring[b], cbase, L, gate, sh_ckey, sh_cpos, sh_var, tid);
          else if (gate >= 0x80000000u)
            gated_append<NT, CAP, 4 * CV, kGatePositive>(ring[b], cbase, L, gate, sh_ckey, sh_cpos, sh_var, tid);
          else
            gated_append<NT, CAP, 4 * CV, kGateAny>(ring[b], cbase, L, gate, sh_ckey, sh_cpos, sh_var, tid);
        }
        load_raw<NT, CV>(ring[b], rowp, kSampleSpan + (idx + NBUF) * kChunkSpan, L, vec, tid);
      }
      __syncthreads();
      if (uniform(sh_var[kVarCandCount]) > kRefresh)
        gate = raise_gate<NT, CAP>(gate, (uint32_t)n, sh_hist, sh_ckey, sh_cpos, sh_scan, sh_var, tid);
    }
    // Every wave's appends are in (the loop's last barrier does this, but a
    // row that fits in the sample has no loop) before the count is read; the
    // histogram is cleared for the list under the same barrier.
    for (int b = tid; b < kBinsWide; b += NT) sh_hist[b] = 0;
    if (tid == 0) sh_var[kVarAbove] = 0;
    __syncthreads();
    // The next row's length and this row's page table are requested now and
    // first used after the finish below.
    int32_t next_len = 0;
    if (tid == 0 && next < (uint32_t)a.batch) next_len = a.seq_lens[next];
    const bool pt_in_lds = PTL && a.pages_per_row <= (int64_t)(4 * NT);
    uint32_t ptv[4];
    if (pt_in_lds) {
      const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<int32_t*>(a.page_table) + (int64_t)row * a.pages_per_row, (short)0,
          (int)(a.pages_per_row * 4), kBufferWord3);
#pragma unroll
      for (int v = 0; v < 4; ++v)
        ptv[v] = __builtin_amdgcn_raw_buffer_load_b32(prs, (uint32_t)tid * 4u, v * NT * 4, 0);
    }

    // 3. The list holds every key >= gate unless it overflowed: its histogram
    // gives the threshold bin, the remaining digits run on the list.  With
    // fewer than n keys at or above the gate (the sample overrated the row)
    // or an overflowed list, the row's histogram is taken from memory (keys
    // below the gate count only in the first case) and the row finished there.
    const uint32_t count = uniform(sh_var[kVarCandCount]);
    const bool low_count = count < (uint32_t)n;
    const bool overflow = low_count || uniform(sh_var[kVarOverflow]) != 0u || count > (uint32_t)CAP;
    const uint32_t floor = low_count ? 1u : gate;
    // The list's keys are all at or above the gate, so their 22-bit prefixes
    // are at or above the gate's, P: a histogram of the prefixes in a window
    // of kBinsWide bins from P (the keys above the window counted apart)
    // resolves the threshold to 22 bits in one pass, where the 12-bit digit
    // needs a 10-bit refinement after it.  When n keys lie above the window
    // (the threshold is above it), the 12-bit histogram is taken instead.
    const uint32_t wbase = gate >> 10;
    bool windowed = false;
    uint32_t above = 0;
    if (!overflow) {
      for (uint32_t i = (uint32_t)tid; i < count; i += NT) {
        const uint32_t d = (sh_ckey[i] >> 10) - wbase;
        if (d < (uint32_t)kBinsWide) atomicAdd(&sh_hist[d], 1u);
        else atomicAdd(&sh_var[kVarAbove], 1u);
      }
      __syncthreads();
      above = uniform(sh_var[kVarAbove]);
      windowed = above < (uint32_t)n;
      if (!windowed) {
        above = 0;
        for (int b = tid; b < kBinsWide; b += NT) sh_hist[b] = 0;
        __syncthreads();
        for (uint32_t i = (uint32_t)tid; i < count; i += NT) atomicAdd(&sh_hist[sh_ckey[i] >> 20], 1u);
        __syncthreads();
      }
    } else {
      for (int b = tid; b < kBinsWide; b += NT) sh_hist[b] = 0;
      __syncthreads();
      restream_pass<NT, CAP, CV>(3, rowp, L, vec, floor, 0u, 20, 0u, (uint32_t)n, sh_hist, sh_ckey, sh_cpos, sh_raw,
                                 sh_var, tid);
    }
    find_threshold<NT, kBinsWide>(sh_hist, (uint32_t)n - above, sh_scan, sh_var, tid);
    const uint32_t t0 = uniform(sh_var[0]), gt0 = uniform(sh_var[1]), cnt0 = uniform(sh_var[2]);
    // From here the first histogram is done with: its upper half holds the
    // selected positions (-1 filled before they are written).
    if (!overflow) {
      // windowed: the threshold's 22-bit prefix, with `above` keys over it
      uint32_t fprefix = windowed ? wbase + t0 : t0, fneed = (uint32_t)n - above - gt0, fcnt = cnt0;
      int fshift = windowed ? 10 : 20;
      // sorted mode: the selected keys go out with the positions (the sorted
      // finish then need not gather them from the row)
      uint32_t* const key_out = a.sel_key ? a.sel_key + row * (int64_t)k : nullptr;
      select_candidates<NT>((int)count, fprefix, fshift, fcnt, fneed, 0u, (uint32_t)n, sh_hist, sh_ckey, sh_cpos,
                            sh_raw, sh_scan, sh_var, tid, true, key_out, a.meta != nullptr);
      if (tid == 0) record_selection(a, row, fprefix, fshift, fneed, fcnt, gate, key_out != nullptr);
    } else {
      for (int j = tid; j < k; j += NT) sh_raw[j] = -1;
      __syncthreads();
      uint32_t prefix = t0, need = (uint32_t)n - gt0, cnt = cnt0;
      int shift = 20;
      while (cnt > (uint32_t)CAP && cnt != need && shift > 0) {
        for (int b = tid; b < kBinsNarrow; b += NT) sh_hist[b] = 0;
        __syncthreads();
        restream_pass<NT, CAP, CV>(0, rowp, L, vec, floor, prefix, shift, need, (uint32_t)n, sh_hist, sh_ckey, sh_cpos,
                                   sh_raw, sh_var, tid);
        find_threshold<NT, kBinsNarrow>(sh_hist, need, sh_scan, sh_var, tid);
        const uint32_t bin = uniform(sh_var[0]), gt = uniform(sh_var[1]);
        cnt = uniform(sh_var[2]);
        need -= gt;
        prefix = (prefix << 10) | bin;
        shift -= 10;
      }
      if (tid == 0) {
        sh_var[kVarGt] = 0;
        sh_var[kVarEq] = 0;
      }
      __syncthreads();
      const bool collect = cnt <= (uint32_t)CAP && cnt != need && shift > 0;
      restream_pass<NT, CAP, CV>(collect ? 1 : 2, rowp, L, vec, floor, prefix, shift, need, (uint32_t)n, sh_hist, sh_ckey,
                                 sh_cpos, sh_raw, sh_var, tid);
      if (collect)
        select_candidates<NT>((int)cnt, prefix, shift, cnt, need, (uint32_t)n - need, (uint32_t)n, sh_hist,
                              sh_ckey, sh_cpos, sh_raw, sh_scan, sh_var, tid, false, nullptr, a.meta != nullptr);
      if (tid == 0) record_selection(a, row, prefix, shift, need, cnt, floor);
    }
    // the candidate list is free again: it holds the page-table row
    int32_t* const sh_pt = reinterpret_cast<int32_t*>(sh_ckey);
    static_assert(!PTL || CAP >= 4 * NT, "the candidate list holds a page-table row of up to 4 NT entries");
    if (pt_in_lds) {
#pragma unroll
      for (int v = 0; v < 4; ++v) sh_pt[tid + v * NT] = (int32_t)ptv[v];
    }
    if (tid == 0) {
      sh_next_row = next;
      sh_next_len = next_len;
    }
    __syncthreads();
    write_row_output<NT>(a, row, L64, n, false, sh_raw, tid, pt_in_lds ? sh_pt : nullptr);
    __syncthreads();
    row = uniform(sh_next_row);
    seq = (int32_t)uniform((uint32_t)sh_next_len);
    if (queue != nullptr) set_row_priority(row, grid);
  }
  // Every workgroup took its last ticket before counting itself out here, so
  // the last one out may reset the queue.
  if (queue != nullptr && threadIdx.x == 0) {
    if (g_add_ret(a.ws + kHdrRowExit, 1u) == grid - 1u) {
      g_store(queue, 0u);
      g_store(a.ws + kHdrRowExit, 0u);
    }
  }
}

// ---------------------------------------------------------------------------
// Split streaming rows (split_stream_kernel): mid batches of long rows.
//
// With fewer rows than CUs, one workgroup per row leaves CUs idle.  Here G
// workgroups share a row (grid = batch * G, every workgroup resident), and
// workgroup g streams the contiguous segment g of the row exactly as the
// streaming kernel streams a whole row: a gate from a sample of its segment
// (ranked for the row's n, so it estimates the row's threshold), the keys at
// or above it appended to an LDS list while the rest of the segment streams
// past, the gate raised when the list fills.  Then, instead of a barrier:
//   * each workgroup writes its list to its own share of the row's area in
//     the workspace, raises the row's floor to its own gate (an atomic max)
//     and flags a list that lost keys;
//   * it counts itself out of the row on one 64-bit word that also sums every
//     part's entry count (each in its own bit field); the last one out
//     finishes the row, with every count in hand.
// Every segment's keys at or above that segment's gate are in the area, so
// the keys at or above the floor (the largest gate) are all there.  If at
// least n of them are, the row's n largest are among them, and the finisher
// selects from its LDS copy exactly as the streaming kernel's finish does.
// Otherwise (fewer than n, or a list lost keys) it finishes the row from
// memory (the streaming kernel's exact fallback).  No workgroup ever waits
// for another, so nothing depends on co-residency.
//
// Per row: four counters in the header, and an area (kSsRowWords words after
// the header) for the appended keys and positions.  The finisher resets the
// counters and zeroes the entries it used, so the workspace is as it was when
// the launch ends.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void g_max(uint32_t* p, uint32_t v) {
  __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// SORTED: the sorted entry point's selection launch (canonical ties, keys
// written beside the positions); a separate instantiation, so that the
// unsorted kernel carries none of that code.
template <int NT, int SV, int CV, int NBUF, int CAP, int WAVES, bool REFINE, bool VEC, bool SORTED>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(WAVES, WAVES)))
split_stream_kernel(KernelArgs a) {
  constexpr uint32_t kSampleSpan = (uint32_t)NT * 4u * SV;
  constexpr uint32_t kChunkSpan = (uint32_t)NT * 4u * CV;
  constexpr uint32_t kRefresh = CAP - CAP / 4;
  constexpr int kLoadPer = (int)(kSsCap / NT);   // area entries per thread the finisher loads at once
  static_assert(CAP >= kBinsNarrow, "the candidate list doubles as the gate's sub-histogram");
  static_assert(kSsCap % NT == 0, "the finisher loads the area in whole rounds");
  static_assert(CAP < (1 << kSsCountBits), "a part's entry count fits its field of the exit word");
  __shared__ uint32_t sh_hist[kBinsWide];
  __shared__ uint32_t sh_ckey[CAP + 1];
  __shared__ int32_t sh_cpos[CAP + 1];
  __shared__ uint32_t sh_scan[64];
  static_assert(kBinsWide - kMaxK >= kBinsNarrow, "selected positions alias the histogram's upper half");
  int32_t* const sh_raw = reinterpret_cast<int32_t*>(sh_hist + (kBinsWide - kMaxK));
  __shared__ uint32_t sh_var[16];

  const int64_t W = a.width;
  const int k = a.k;
  constexpr bool vec = VEC;
  int G = a.wgs_per_row;
  int64_t row;
  uint32_t part;
  int32_t seq;
  // Part `part` of G of a row of Lx positions: [a0, a1), whole multiples of
  // one float4 per thread, so every segment starts 16-byte aligned.
  auto segment = [&](uint32_t Lx, uint32_t& a0, uint32_t& a1) {
    const uint32_t per = (Lx + (uint32_t)G - 1u) / (uint32_t)G;
    const uint32_t seglen = (per + 4u * NT - 1u) / (4u * NT) * (4u * NT);
    a0 = part * seglen < Lx ? part * seglen : Lx;
    a1 = Lx - a0 > seglen ? a0 + seglen : Lx;
  };
  // The sample's loads are issued before the row's length is read, for the
  // segment of a row as long as the width (the usual case); they are issued
  // again for the real segment if it differs.
  uint32_t sk[4 * SV];
  uint32_t s0w = 1u, s1w = 0u;   // the speculative segment (none for length-aware parts)
  if (a.spread == 0) {   // G parts for every row
    row = (int64_t)(blockIdx.x / (uint32_t)G);
    part = blockIdx.x - (uint32_t)row * (uint32_t)G;
    if (row >= a.batch) return;
    segment((uint32_t)W, s0w, s1w);
    load_raw<NT, SV>(sk, a.scores + row * W, s0w, s1w, vec, opaque_tid());
    seq = scalar_read(a.seq_lens, row);
  } else {
    // Length-aware: every workgroup reads the batch's lengths (at most
    // kSsMaxRows rows) and gives row r G_r = ceil(L_r / T) parts, between 1
    // and G, with T the batch's positions over `spread` shares (about one
    // workgroup per CU); rows of at most k positions get one.  Workgroups are
    // numbered through the rows in order, parts within a row; those past the
    // total exit.  The grid is batch * G.
    const int t = opaque_tid();
    int32_t sl = t < a.batch ? a.seq_lens[t] : 0;
    const uint32_t Lt = sl <= 0 ? 0u : ((int64_t)sl > W ? (uint32_t)W : (uint32_t)sl);
    uint32_t kilo_total;   // the batch's positions, in units of 1024 (fits 32 bits for 256 rows)
    block_exclusive_scan<NT>(Lt >> 10, sh_scan, kilo_total, t);
    const uint32_t share = (kilo_total + (uint32_t)a.spread - 1u) / (uint32_t)a.spread * 1024u;   // T
    uint32_t gt = 0u;
    if (t < a.batch) {
      gt = 1u;
      if (Lt > (uint32_t)k && share > 0u) {
        const uint32_t want = (Lt + share - 1u) / share;
        gt = want < 1u ? 1u : (want > (uint32_t)G ? (uint32_t)G : want);
      }
    }
    uint32_t units;
    const uint32_t first = block_exclusive_scan<NT>(gt, sh_scan, units, t);
    if (t < a.batch && blockIdx.x >= first && blockIdx.x < first + gt) {
      sh_var[0] = (uint32_t)t;
      sh_var[1] = blockIdx.x - first;
      sh_var[2] = gt;
      sh_var[3] = (uint32_t)sl;
    }
    __syncthreads();
    if (blockIdx.x >= units) return;
    row = (int64_t)uniform(sh_var[0]);
    part = uniform(sh_var[1]);
    G = (int)uniform(sh_var[2]);
    seq = (int32_t)uniform(sh_var[3]);
    __syncthreads();   // sh_var is reused below
  }
  const int tid = opaque_tid();
  const int64_t L64 = seq < 0 ? 0 : ((int64_t)seq > W ? W : (int64_t)seq);
  const uint32_t L = (uint32_t)L64;
  const int n = L64 < (int64_t)k ? (int)L64 : k;
  if (L64 <= (int64_t)k) {   // every valid position is selected; the row's area is not used
    if (part == 0u) {
      write_row_output<NT>(a, row, L64, n, true, sh_raw, tid);
      if (tid == 0) record_selection(a, row, 0u, 32, (uint32_t)n, (uint32_t)n, 0u);
    }
    return;
  }
  uint32_t s0, s1;   // this part's segment
  segment(L, s0, s1);
  uint32_t* const ctr = a.ws + kSsCtr + 4 * (size_t)row;
  uint32_t* const area = a.ws + kHdrWords + (size_t)row * kSsRowWords;
  const float* rowp = a.scores + row * W;

  for (int b = tid; b < kBinsWide; b += NT) sh_hist[b] = 0;
  if (tid < 16) sh_var[tid] = 0;
  __syncthreads();
  uint32_t gate = 0u;
  if (s0 < s1) {
    // 1. sample: the first kSampleSpan positions of the segment
    if (s0 != s0w || s1 != s1w) load_raw<NT, SV>(sk, rowp, s0, s1, vec, tid);
    const uint32_t seg = s1 - s0;
    const uint32_t nch = seg > kSampleSpan ? (seg - kSampleSpan + kChunkSpan - 1) / kChunkSpan : 0u;
#pragma unroll
    for (int j = 0; j < 4 * SV; ++j) {
      const uint32_t x = slot_key<NT>(sk[j], j, s0, s1, tid);
      if (x) atomicAdd(&sh_hist[x >> 20], 1u);
    }
    __syncthreads();
    // The first chunks are requested only now: every workgroup of the launch
    // starts at once, and samples requested alone arrive sooner; these loads
    // then stream in while the gate is worked out.  As in the streaming
    // kernel, every ring load is issued (past the segment they read nothing),
    // so that each chunk's use waits for that chunk only.
    uint32_t ring[NBUF][4 * CV];
#pragma unroll
    for (int b = 0; b < NBUF; ++b)
      load_raw<NT, CV>(ring[b], rowp, s0 + kSampleSpan + (uint32_t)b * kChunkSpan, s1, vec, tid);
    // ranked for the row: the sample holds on average n * S / L of the row's n largest
    const uint32_t m = gate_rank((uint32_t)n, seg < kSampleSpan ? seg : kSampleSpan, L);
    find_threshold<NT, kBinsWide>(sh_hist, m, sh_scan, sh_var, tid);
    const uint32_t gbin = uniform(sh_var[0]), gneed = m - uniform(sh_var[1]);
    gate = gbin << 20;
    if (REFINE) {   // the gate refined inside its bin with the next 10 key bits
      for (int b = tid; b < kBinsNarrow; b += NT) sh_ckey[b] = 0u;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 4 * SV; ++j) {
        const uint32_t x = slot_key<NT>(sk[j], j, s0, s1, tid);
        if (x != 0u && (x >> 20) == gbin) atomicAdd(&sh_ckey[(x >> 10) & 1023u], 1u);
      }
      __syncthreads();
      find_threshold<NT, kBinsNarrow>(sh_ckey, gneed, sh_scan, sh_var, tid);
      gate |= uniform(sh_var[0]) << 10;
    }
    if (gate == 0u) gate = 1u;
    {
      static_assert(SV % 2 == 0, "the sample is appended in two halves");
      uint32_t lo[2 * SV], hi[2 * SV];
#pragma unroll
      for (int j = 0; j < 2 * SV; ++j) {
        lo[j] = sk[j];
        hi[j] = sk[2 * SV + j];
      }
      constexpr uint32_t half = (uint32_t)NT * 4u * (SV / 2);
      gated_append<NT, CAP, 2 * SV, kGateChecked>(lo, s0, s1, gate, sh_ckey, sh_cpos, sh_var, tid);
      gated_append<NT, CAP, 2 * SV, kGateChecked>(hi, s0 + half, s1, gate, sh_ckey, sh_cpos, sh_var, tid);
    }
    // 2. stream the rest of the segment through the ring
    for (uint32_t i = 0; i < nch; i += NBUF) {
#pragma unroll
      for (int b = 0; b < NBUF; ++b) {
        const uint32_t idx = i + (uint32_t)b;
        if (idx < nch) {
          const uint32_t cbase = s0 + kSampleSpan + idx * kChunkSpan;
          if (cbase + kChunkSpan > s1)
            gated_append<NT, CAP, 4 * CV, kGateChecked>(ring[b], cbase, s1, gate, sh_ckey, sh_cpos, sh_var, tid);
          else if (gate >= 0x80000000u)
            gated_append<NT, CAP, 4 * CV, kGatePositive>(ring[b], cbase, s1, gate, sh_ckey, sh_cpos, sh_var, tid);
          else
            gated_append<NT, CAP, 4 * CV, kGateAny>(ring[b], cbase, s1, gate, sh_ckey, sh_cpos, sh_var, tid);
        }
        load_raw<NT, CV>(ring[b], rowp, s0 + kSampleSpan + (idx + NBUF) * kChunkSpan, s1, vec, tid);
      }
      __syncthreads();
      if (uniform(sh_var[kVarCandCount]) > kRefresh)
        gate = raise_gate<NT, CAP>(gate, (uint32_t)n, sh_hist, sh_ckey, sh_cpos, sh_scan, sh_var, tid);
    }
  }
  __syncthreads();   // every wave's appends are in

  // 3. publish the segment's list (keys >= gate, all of them unless it lost
  // some) in the part's own share of the row's area, then count out on the
  // row's exit word, which also carries every part's entry count.
  const uint32_t partcap = (uint32_t)kSsCap / (uint32_t)G;
  {
    const uint32_t count = uniform(sh_var[kVarCandCount]);
    const uint32_t ncur = count < (uint32_t)CAP ? count : (uint32_t)CAP;
    const uint32_t nput = ncur < partcap ? ncur : partcap;
    const bool lost = uniform(sh_var[kVarOverflow]) != 0u || count > (uint32_t)CAP || ncur > partcap;
    for (uint32_t i = (uint32_t)tid; i < nput; i += NT) {
      g_store(area + kSsKeys + part * partcap + i, sh_ckey[i]);
      g_store(area + kSsPos + part * partcap + i, (uint32_t)sh_cpos[i]);
    }
    if (tid == 0) {
      if (gate != 0u) g_max(ctr + kSsFloor, gate);
      if (lost) g_store(ctr + kSsFlag, 1u);
    }
    wave_mem_drain();
    __syncthreads();
    if (tid == 0) {
      const uint64_t mine = 1ull | ((uint64_t)nput << (kSsExitBits + kSsCountBits * part));
      const uint64_t all = g_add64_ret(reinterpret_cast<uint64_t*>(ctr + kSsExit), mine) + mine;
      const bool last = (uint32_t)(all & ((1ull << kSsExitBits) - 1ull)) == (uint32_t)G;
      sh_var[4] = last ? 1u : 0u;
#pragma unroll
      for (int g = 0; g < kSsMaxParts; ++g)
        sh_var[5 + g] = (uint32_t)(all >> (kSsExitBits + kSsCountBits * g)) & ((1u << kSsCountBits) - 1u);
    }
    __syncthreads();
    if (uniform(sh_var[4]) == 0u) return;
  }

  // 4. the last workgroup out finishes the row.  Every other workgroup drained
  // its appends and its floor before counting itself out; the exit word gave
  // every part's count, so the floor, the flag and the entries are requested
  // together.
  uint32_t pc[kSsMaxParts], pstart[kSsMaxParts + 1];
  pstart[0] = 0u;
#pragma unroll
  for (int g = 0; g < kSsMaxParts; ++g) {
    pc[g] = g < G ? uniform(sh_var[5 + g]) : 0u;
    pstart[g + 1] = pstart[g] + pc[g];
  }
  const uint32_t nload = pstart[kSsMaxParts];
  uint32_t xk[kLoadPer], xp[kLoadPer];
#pragma unroll
  for (int r = 0; r < kLoadPer; ++r) {
    const uint32_t i = (uint32_t)tid + (uint32_t)r * NT;
    uint32_t g = 0;
#pragma unroll
    for (int q = 1; q < kSsMaxParts; ++q) g += i >= pstart[q] ? 1u : 0u;
    const uint32_t at = g * partcap + (i - pstart[g]);
    xk[r] = i < nload ? g_load(area + kSsKeys + at) : 0u;
    xp[r] = i < nload ? g_load(area + kSsPos + at) : 0u;
  }
  const uint32_t floor0 = g_load(ctr + kSsFloor);   // >= 1: the row has a nonempty segment
  const bool lost = g_load(ctr + kSsFlag) != 0u;
  if (tid == 0) {
    sh_var[kVarCandCount] = 0u;
    sh_var[kVarOverflow] = 0u;
    sh_var[kVarAbove] = 0u;
  }
  for (int b = tid; b < kBinsWide; b += NT) sh_hist[b] = 0;
  __syncthreads();
  // As the keys are appended, their 22-bit prefixes are counted in a window
  // of kBinsWide bins from the floor's (keys above it counted apart), as in
  // the streaming finish: the threshold comes out at 22 bits from one pass.
  const uint32_t wbase = floor0 >> 10;
  {
    // the area's keys >= floor into the LDS list: one ballot append per round
    const int lane = tid & 63;
#pragma unroll
    for (int r = 0; r < kLoadPer; ++r) {
      const bool pass = xk[r] >= floor0 && xk[r] != 0u;
      const uint64_t msk = __ballot(pass);
      if (msk == 0ull) continue;
      uint32_t lbase = 0;
      if (lane == 0) lbase = atomicAdd(&sh_var[kVarCandCount], (uint32_t)__popcll(msk));
      lbase = __builtin_amdgcn_readfirstlane(lbase);
      if (pass) {
        uint32_t slot = lbase + lanes_below(msk);
        slot = slot < (uint32_t)CAP ? slot : (uint32_t)CAP;
        sh_ckey[slot] = xk[r];
        sh_cpos[slot] = (int32_t)xp[r];
        const uint32_t d = (xk[r] >> 10) - wbase;
        if (d < (uint32_t)kBinsWide) atomicAdd(&sh_hist[d], 1u);
        else atomicAdd(&sh_var[kVarAbove], 1u);
      }
    }
  }
  __syncthreads();
  const uint32_t count = uniform(sh_var[kVarCandCount]);
  const bool low_count = count < (uint32_t)n;
  const bool overflow = lost || low_count || count > (uint32_t)CAP;
  const uint32_t floor = low_count ? 1u : floor0;
  uint32_t above = overflow ? 0u : uniform(sh_var[kVarAbove]);
  const bool windowed = !overflow && above < (uint32_t)n;
  if (!windowed) {   // the 12-bit histogram instead: of the list, or of the row from memory
    above = 0;
    for (int b = tid; b < kBinsWide; b += NT) sh_hist[b] = 0;
    __syncthreads();
    if (!overflow) {
      for (uint32_t i = (uint32_t)tid; i < count; i += NT) atomicAdd(&sh_hist[sh_ckey[i] >> 20], 1u);
      __syncthreads();
    } else {
      restream_pass<NT, CAP, CV>(3, rowp, L, vec, floor, 0u, 20, 0u, (uint32_t)n, sh_hist, sh_ckey, sh_cpos, sh_raw,
                                 sh_var, tid);
    }
  }
  find_threshold<NT, kBinsWide>(sh_hist, (uint32_t)n - above, sh_scan, sh_var, tid);
  const uint32_t t0 = uniform(sh_var[0]), gt0 = uniform(sh_var[1]), cnt0 = uniform(sh_var[2]);
  if (!overflow) {
    // windowed: the threshold's 22-bit prefix, with `above` keys over it
    uint32_t fprefix = windowed ? wbase + t0 : t0, fneed = (uint32_t)n - above - gt0, fcnt = cnt0;
    int fshift = windowed ? 10 : 20;
    // sorted mode: the selected keys go out with the positions
    uint32_t* const key_out = SORTED && a.sel_key ? a.sel_key + row * (int64_t)k : nullptr;
    select_candidates<NT>((int)count, fprefix, fshift, fcnt, fneed, 0u, (uint32_t)n, sh_hist, sh_ckey, sh_cpos,
                          sh_raw, sh_scan, sh_var, tid, true, key_out, SORTED);
    if (tid == 0) record_selection(a, row, fprefix, fshift, fneed, fcnt, floor, key_out != nullptr);
  } else {
    for (int j = tid; j < k; j += NT) sh_raw[j] = -1;
    __syncthreads();
    uint32_t prefix = t0, need = (uint32_t)n - gt0, cnt = cnt0;
    int shift = 20;
    while (cnt > (uint32_t)CAP && cnt != need && shift > 0) {
      for (int b = tid; b < kBinsNarrow; b += NT) sh_hist[b] = 0;
      __syncthreads();
      restream_pass<NT, CAP, CV>(0, rowp, L, vec, floor, prefix, shift, need, (uint32_t)n, sh_hist, sh_ckey, sh_cpos,
                                 sh_raw, sh_var, tid);
      find_threshold<NT, kBinsNarrow>(sh_hist, need, sh_scan, sh_var, tid);
      const uint32_t bin = uniform(sh_var[0]), gt = uniform(sh_var[1]);
      cnt = uniform(sh_var[2]);
      need -= gt;
      prefix = (prefix << 10) | bin;
      shift -= 10;
    }
    if (tid == 0) {
      sh_var[kVarGt] = 0;
      sh_var[kVarEq] = 0;
    }
    __syncthreads();
    const bool collect = cnt <= (uint32_t)CAP && cnt != need && shift > 0;
    restream_pass<NT, CAP, CV>(collect ? 1 : 2, rowp, L, vec, floor, prefix, shift, need, (uint32_t)n, sh_hist, sh_ckey,
                               sh_cpos, sh_raw, sh_var, tid);
    if (collect)
      select_candidates<NT>((int)cnt, prefix, shift, cnt, need, (uint32_t)n - need, (uint32_t)n, sh_hist, sh_ckey,
                            sh_cpos, sh_raw, sh_scan, sh_var, tid, false, nullptr, SORTED);
    if (tid == 0) record_selection(a, row, prefix, shift, need, cnt, floor);
  }
  __syncthreads();
  write_row_output<NT>(a, row, L64, n, false, sh_raw, tid);
  // leave the row's area and counters zeroed
#pragma unroll
  for (int g = 0; g < kSsMaxParts; ++g)
    for (uint32_t i = (uint32_t)tid; i < pc[g]; i += NT) {
      g_store(area + kSsKeys + (uint32_t)g * partcap + i, 0u);
      g_store(area + kSsPos + (uint32_t)g * partcap + i, 0u);
    }
  if (tid < 4) g_store(ctr + tid, 0u);
}

// ---------------------------------------------------------------------------
// Sorted finish (deterministic mode).
//
// A selection launch recorded, per row, how its threshold ended
// (record_selection).  This kernel streams the row once more and rewrites the
// row's outputs in the canonical order: key descending, equal keys by position
// ascending, and where the threshold bin is cut, the tied positions taken are
// the lowest.  That is the order the plain definition gives (sort by key
// descending, then position ascending, take the first n), so the output is
// unique: equal for every kernel shape, every run.
//
// Per row: when the record says the final bin was not cut, the selection
// launch's positions (`sel`) are already the canonical set: their keys are
// gathered from the row and the pairs sorted, with no second read of the row.
// Otherwise the keys above the final bin (exactly n - need of them) go to
// sh_sort; the bin's members go to a tie list.  When the bin holds more than
// `need`, the `need` lowest positions are found by an MSB-first radix select
// on v = ~position (the largest v are the lowest positions; positions are
// distinct, so it ends with the bin holding exactly what is needed).  If more
// members than the tie list holds, the same select runs over the row in
// memory.  The n chosen (key, ~position) pairs are then bitonic-sorted in LDS.
// ---------------------------------------------------------------------------
// float4 groups per thread per streamed chunk: 64 KB of the row per chunk for
// 512 threads and more; 16 KB for the 256-thread shape, whose registers set
// how many workgroups a CU holds
template <int NT>
constexpr int sort_cv() { return NT >= 512 ? 4096 / NT : 4; }

// Histogram bins of the sorted finish (the rank finish's buckets, the cut
// rows' tie select): 1024 for the small shape (k <= kSortSmallK), whose LDS
// sets how many workgroups a CU holds, else 4096.
template <int CAP>
constexpr int sort_hist_bins() { return CAP <= kSortSmallK ? kBinsNarrow : kBinsWide; }

// One pass over the row for the memory fallback of the tie select: with
// `collect` false, histograms the digit (v >> dshift) & dmask of v =
// ~position of the bin members whose v >> (vshift) == vprefix (vshift 32:
// all); with `collect` true, appends the members with v >> vshift >= vprefix
// to sh_sort from slot `base` on.
template <int NT, int CAP>
__device__ __forceinline__ void sorted_tie_pass(bool collect, const float* rowp, uint32_t L, bool vec,
                                                uint32_t prefix, int shift, uint32_t floor, uint32_t vprefix,
                                                int vshift, int dshift, uint32_t dmask, uint32_t* sh_hist,
                                                uint64_t* sh_sort, uint32_t base, uint32_t* sh_var, int tid) {
  constexpr uint32_t span = (uint32_t)NT * 4u * sort_cv<NT>();
  for (uint32_t c = 0; c < L; c += span) {
    uint32_t raw[4 * sort_cv<NT>()];
    load_raw<NT, sort_cv<NT>(), kLoadReuse>(raw, rowp, c, L, vec, tid);
#pragma unroll
    for (int j = 0; j < 4 * sort_cv<NT>(); ++j) {
      const uint32_t pos = c + (uint32_t)tid * 4u + (uint32_t)(j >> 2) * (NT * 4) + (uint32_t)(j & 3);
      if (pos >= L) continue;
      const uint32_t x = order_key_bits(raw[j]);
      if (x < floor || ((uint64_t)x >> shift) != (uint64_t)prefix) continue;
      const uint32_t v = ~pos;
      const uint32_t vp = vshift >= 32 ? 0u : v >> vshift;
      if (!collect) {
        if (vshift >= 32 || vp == vprefix) atomicAdd(&sh_hist[(v >> dshift) & dmask], 1u);
      } else if (vp >= vprefix) {
        const uint32_t s = base + atomicAdd(&sh_var[2], 1u);
        if (s < (uint32_t)CAP) sh_sort[s] = ((uint64_t)x << 32) | (uint64_t)v;
      }
    }
  }
  __syncthreads();
}

// Sorts a row's pairs sh_sort[0, n) descending with a bitonic network over
// the next power of two P >= n (sh_sort[n, P) must hold distinct pads below
// every pair, e.g. their indices), then writes the row's k output slots:
// slot j < n the position of pair j (-1 if not below L) transformed through
// the page table, the rest -1.  Contains barriers: call uniformly.
template <int NT>
__device__ void bitonic_write(const KernelArgs& a, int64_t row, uint32_t n, uint32_t L, uint64_t* sh_sort, int tid) {
  const int k = a.k;
  uint32_t P = 1;
  while (P < n) P <<= 1;
  for (uint32_t size = 2; size <= P; size <<= 1) {
    for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
      for (uint32_t i = (uint32_t)tid; i < P / 2; i += NT) {
        const uint32_t lo = 2 * i - (i & (stride - 1));
        const uint32_t hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint64_t x = sh_sort[lo], y = sh_sort[hi];
        if ((x < y) == desc) {
          sh_sort[lo] = y;
          sh_sort[hi] = x;
        }
      }
      __syncthreads();
    }
  }
  const int s = a.log2_page;
  const uint32_t pmask = (1u << s) - 1u;
  int32_t* o = a.out + row * (int64_t)k;
  int32_t* orw = a.out_raw ? a.out_raw + row * (int64_t)k : nullptr;
  const int32_t* pt = a.page_table + row * a.pages_per_row;
  for (int j = tid; j < k; j += NT) {
    int32_t r = -1, v = -1;
    if ((uint32_t)j < n) {
      const uint32_t p = ~(uint32_t)sh_sort[j];
      if (p < L) {
        r = (int32_t)p;
        const int64_t pg = (int64_t)(p >> s);
        if (pg < a.pages_per_row) v = (int32_t)(((uint32_t)pt[pg] << s) | (p & pmask));
      }
    }
    o[j] = v;
    if (orw) orw[j] = r;
  }
}

// Prepares rank_pairs_write's inputs for pairs that thread tid saw (hi, lo:
// the largest and smallest of them; lo > hi if none): sh_mm = {Pmax, Pmin}
// of the workgroup.  sh_mm must hold {0, ~0} beforehand (pairs_span_init,
// then a barrier); ends with a barrier.
__device__ __forceinline__ void pairs_span(uint64_t hi, uint64_t lo, uint64_t* sh_mm, int tid) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t h2 = ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(hi >> 32), off, 64) << 32) |
                        (uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)hi, off, 64);
    const uint64_t l2 = ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(lo >> 32), off, 64) << 32) |
                        (uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)lo, off, 64);
    hi = h2 > hi ? h2 : hi;
    lo = l2 < lo ? l2 : lo;
  }
  if ((tid & 63) == 0 && lo <= hi) {
    atomicMax(reinterpret_cast<unsigned long long*>(&sh_mm[0]), (unsigned long long)hi);
    atomicMin(reinterpret_cast<unsigned long long*>(&sh_mm[1]), (unsigned long long)lo);
  }
  __syncthreads();
}

// Zeroes rank_pairs_write's bucket counts and resets its span and largest
// bucket words (a barrier must follow before pairs_span).
template <int NT, int NB>
__device__ __forceinline__ void pairs_span_init(uint32_t* sh_cnt, uint64_t* sh_mm, uint32_t* sh_scan, int tid) {
  for (int b = tid; b < NB; b += NT) sh_cnt[b] = 0;
  if (tid == 0) {
    sh_mm[0] = 0ull;
    sh_mm[1] = ~0ull;
    sh_scan[48] = 0;   // the largest bucket (a block scan uses sh_scan[0, NT/64])
  }
}

// Writes pairs sh_a[j0, j1) of a row's n distinct pairs P = (key << 32) |
// ~position (sh_a[0, n) filled and visible) to their slots in the canonical
// order: slot = rank = #{P' > P}, transformed through the page table; a pair
// whose position is not below L is written as -1.  The pairs are grouped into
// NB buckets by (P - Pmin) >> s, s chosen so that the row's span Pmax - Pmin
// fills the buckets (a monotone map: each bucket is a range of P); a rank is
// then the number of pairs in higher buckets plus a count over the pair's own
// bucket, split over up to 64 threads per pair.
//
// A bucket of more than kRankMaxBucket pairs (many equal keys: the pairs of
// one key differ only in their positions, and when the row's span is set by
// other keys they share a bucket) is split once more, by kSubBins
// sub-buckets fitted to its own span (for equal keys, the positions' span),
// and its pairs are ranked within their sub-bucket.  Returns false, having
// written nothing and with sh_a[0, n) holding the row's pairs again, when a
// sub-bucket is still crowded; the caller then orders the row otherwise.
//
// sh_b holds n pairs, sh_beg and sh_cnt NB words each, sh_sub kSubWords
// words, sh_mm2 two.  On entry (after a barrier) sh_mm = {Pmax, Pmin},
// sh_cnt is zero and sh_scan[48] is zero (see pairs_span).  sh_a is
// scratch once the pairs are grouped.  Contains barriers: call uniformly.
constexpr uint32_t kRankMaxBucket = 256;
constexpr int kSubBins = 256;
constexpr int kRankMaxCrowded = 8;   // > n / (kRankMaxBucket + 1) for n <= kMaxK
constexpr int kSubCnt = 0, kSubBeg = kSubBins, kSubCrowdN = 2 * kSubBins, kSubBig = kSubCrowdN + 1,
              kSubCrowd = kSubBig + 1, kSubWords = kSubCrowd + kRankMaxCrowded;
template <int NT, int NB, int CAP>
__device__ bool rank_pairs_write(const KernelArgs& a, int64_t row, uint32_t n, uint32_t L, uint32_t j0, uint32_t j1,
                                 uint64_t* sh_a, uint64_t* sh_b, uint32_t* sh_beg, uint32_t* sh_cnt,
                                 uint64_t* sh_mm, uint32_t* sh_scan, uint32_t* sh_sub, uint64_t* sh_mm2, int tid) {
  constexpr int kDigit = NB == 4096 ? 12 : (NB == 2048 ? 11 : (NB == 1024 ? 10 : -1));
  static_assert(kDigit > 0 && NB % NT == 0, "rank digit");
  static_assert(NT >= kSubBins, "one sub-bucket per thread");
  const int k = a.k;
  // 1. this thread's pairs (e = j0 + it * per + tid / tpe, tpe threads per
  // pair), held in registers since sh_a becomes scratch, and their page-table
  // entries requested before any rank is counted (so the output's gather
  // overlaps the counting).  A thread handles at most CAP / NT pairs: tpe = 1
  // gives ceil(cnt / NT) rounds, a larger tpe one round.
  const uint32_t cnt_here = j1 - j0;
  uint32_t tpe = 64;
  while (tpe > 1 && tpe * cnt_here > (uint32_t)NT) tpe >>= 1;
  const uint32_t per = (uint32_t)NT / tpe;
  const uint32_t q = (uint32_t)tid & (tpe - 1u);
  const int s = a.log2_page;
  const uint32_t pmask = (1u << s) - 1u;
  const int32_t* pt = a.page_table + row * a.pages_per_row;
  constexpr int kRounds = CAP / NT;
  uint64_t mine[kRounds];
  int32_t page[kRounds];
  uint32_t rk[kRounds];   // ranks of pairs in refined buckets (lane q == 0)
#pragma unroll
  for (int it = 0; it < kRounds; ++it) {
    const uint32_t e = j0 + (uint32_t)it * per + (uint32_t)tid / tpe;
    mine[it] = e < j1 ? sh_a[e] : 0ull;
    page[it] = 0;
    rk[it] = 0u;
    if (e < j1 && q == 0) {
      const uint32_t p = ~(uint32_t)mine[it];
      if (p < L && (int64_t)(p >> s) < a.pages_per_row) page[it] = pt[p >> s];
    }
  }

  // 2. bucket counts
  const uint64_t pmin = sh_mm[1];
  const uint64_t range = sh_mm[0] - pmin;
  const int top = range != 0ull ? 63 - __builtin_clzll(range) : 0;
  const int bs = top >= kDigit - 1 ? top - (kDigit - 1) : 0;
  auto bucket = [&](uint64_t P) { return (uint32_t)((P - pmin) >> bs) & (uint32_t)(NB - 1); };
  if (tid == 0) sh_sub[kSubCrowdN] = 0u;
  for (uint32_t j = (uint32_t)tid; j < n; j += NT) atomicAdd(&sh_cnt[bucket(sh_a[j])], 1u);
  __syncthreads();

  // 3. first slots, buckets in descending order: thread t owns buckets
  // NB-1-(NB/NT)t down to NB-(NB/NT)(t+1); crowded buckets are listed
  {
    constexpr int kPer = NB / NT;
    uint32_t c[kPer], sum = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      c[i] = sh_cnt[NB - 1 - kPer * tid - i];
      sum += c[i];
      if (c[i] > kRankMaxBucket) {
        const uint32_t slot = atomicAdd(&sh_sub[kSubCrowdN], 1u);
        if (slot < (uint32_t)kRankMaxCrowded) sh_sub[kSubCrowd + slot] = (uint32_t)(NB - 1 - kPer * tid - i);
      }
    }
    uint32_t total;
    uint32_t run = block_exclusive_scan<NT>(sum, sh_scan, total, tid);   // ends with a barrier
    if (uniform(sh_sub[kSubCrowdN]) > (uint32_t)kRankMaxCrowded) return false;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      sh_beg[NB - 1 - kPer * tid - i] = run;
      run += c[i];
    }
  }
  __syncthreads();

  // 4. group the pairs by bucket (order within a bucket does not matter); the
  // cursors end one past each bucket, so the first slots are end - count
  for (uint32_t j = (uint32_t)tid; j < n; j += NT) {
    const uint64_t P = sh_a[j];
    sh_b[atomicAdd(&sh_beg[bucket(P)], 1u)] = P;
  }
  __syncthreads();

  // 5. crowded buckets, one at a time: sub-buckets fitted to the bucket's
  // span, the bucket's pairs regrouped by sub-bucket (descending) in place,
  // and the ranks of this thread's pairs in it counted over their sub-bucket
  const uint32_t ncrowd = uniform(sh_sub[kSubCrowdN]);
  for (uint32_t ci = 0; ci < ncrowd; ++ci) {
    const uint32_t b = uniform(sh_sub[kSubCrowd + ci]);
    const uint32_t bend = sh_beg[b], bfirst = bend - sh_cnt[b];
    if (tid == 0) {
      sh_mm2[0] = 0ull;
      sh_mm2[1] = ~0ull;
      sh_sub[kSubBig] = 0u;
    }
    if (tid < kSubBins) sh_sub[kSubCnt + tid] = 0u;
    __syncthreads();
    uint64_t hi = 0ull, lo = ~0ull;
    for (uint32_t i = bfirst + (uint32_t)tid; i < bend; i += NT) {
      const uint64_t P = sh_b[i];
      hi = P > hi ? P : hi;
      lo = P < lo ? P : lo;
    }
    pairs_span(hi, lo, sh_mm2, tid);
    const uint64_t smin = sh_mm2[1];
    const uint64_t srange = sh_mm2[0] - smin;
    const int stop = srange != 0ull ? 63 - __builtin_clzll(srange) : 0;
    const int sbs = stop >= 7 ? stop - 7 : 0;   // kSubBins = 2^8
    auto sub = [&](uint64_t P) { return (uint32_t)((P - smin) >> sbs) & (uint32_t)(kSubBins - 1); };
    for (uint32_t i = bfirst + (uint32_t)tid; i < bend; i += NT) atomicAdd(&sh_sub[kSubCnt + sub(sh_b[i])], 1u);
    __syncthreads();
    // descending sub-bucket starts (relative to bfirst); thread t owns sub-bucket kSubBins-1-t
    const uint32_t sc = tid < kSubBins ? sh_sub[kSubCnt + kSubBins - 1 - tid] : 0u;
    uint32_t big = sc;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const uint32_t o2 = (uint32_t)__shfl_xor((int)big, off, 64);
      big = o2 > big ? o2 : big;
    }
    if ((tid & 63) == 0) atomicMax(&sh_sub[kSubBig], big);
    uint32_t total;
    const uint32_t srun = block_exclusive_scan<NT>(sc, sh_scan, total, tid);   // ends with a barrier
    if (uniform(sh_sub[kSubBig]) > kRankMaxBucket) {
      // still crowded: hand the caller the row's pairs back in sh_a
      for (uint32_t j = (uint32_t)tid; j < n; j += NT) sh_a[j] = sh_b[j];
      __syncthreads();
      return false;
    }
    if (tid < kSubBins) sh_sub[kSubBeg + kSubBins - 1 - tid] = srun;
    for (uint32_t i = bfirst + (uint32_t)tid; i < bend; i += NT) sh_a[i] = sh_b[i];
    __syncthreads();
    for (uint32_t i = bfirst + (uint32_t)tid; i < bend; i += NT) {
      const uint64_t P = sh_a[i];
      sh_b[bfirst + atomicAdd(&sh_sub[kSubBeg + sub(P)], 1u)] = P;
    }
    __syncthreads();
    // the cursors end one past each sub-bucket
#pragma unroll
    for (int it = 0; it < kRounds; ++it) {
      const uint32_t e = j0 + (uint32_t)it * per + (uint32_t)tid / tpe;
      const uint64_t P = mine[it];
      if (e < j1 && q == 0 && bucket(P) == b) {
        const uint32_t sb = sub(P);
        const uint32_t send = bfirst + sh_sub[kSubBeg + sb], sfirst = send - sh_sub[kSubCnt + sb];
        uint32_t c = 0;
        for (uint32_t i = sfirst; i < send; ++i) c += sh_b[i] > P ? 1u : 0u;
        rk[it] = sfirst + c;
      }
    }
    __syncthreads();
  }

  // 6. ranks of pairs [j0, j1), tpe threads per pair, and the output
  int32_t* o = a.out + row * (int64_t)k;
  int32_t* orw = a.out_raw ? a.out_raw + row * (int64_t)k : nullptr;
#pragma unroll
  for (int it = 0; it < kRounds; ++it) {
    const uint32_t base = (uint32_t)it * per;
    if (base >= cnt_here) break;   // uniform
    const uint32_t e = j0 + base + (uint32_t)tid / tpe;
    const bool act = e < j1;
    const uint64_t P = mine[it];
    uint32_t first = 0, c = 0;
    bool refined = false;
    if (act) {
      const uint32_t b = bucket(P);
      refined = sh_cnt[b] > kRankMaxBucket;
      if (!refined) {
        const uint32_t end = sh_beg[b];
        first = end - sh_cnt[b];
        uint32_t i = first + q;
        for (; i + 3u * tpe < end; i += 4u * tpe) {   // four independent reads in flight
          const uint64_t b0 = sh_b[i], b1 = sh_b[i + tpe], b2 = sh_b[i + 2u * tpe], b3 = sh_b[i + 3u * tpe];
          c += (b0 > P ? 1u : 0u) + (b1 > P ? 1u : 0u) + (b2 > P ? 1u : 0u) + (b3 > P ? 1u : 0u);
        }
        for (; i < end; i += tpe) c += sh_b[i] > P ? 1u : 0u;
      }
    }
    for (uint32_t off = 1; off < tpe; off <<= 1) c += (uint32_t)__shfl_xor((int)c, (int)off, 64);
    if (act && q == 0) {
      const uint32_t r = refined ? rk[it] : first + c;
      const uint32_t p = ~(uint32_t)P;
      int32_t rv = -1, v = -1;
      if (p < L) {
        rv = (int32_t)p;
        if ((int64_t)(p >> s) < a.pages_per_row) v = (int32_t)(((uint32_t)page[it] << s) | (p & pmask));
      }
      o[r] = v;
      if (orw) orw[r] = rv;
    }
  }
  return true;
}

// The sorted finish of one row by one NT-thread workgroup (contains barriers:
// call uniformly).  sh_sort holds CAP pairs, sh_tk / sh_tp TIES entries each,
// sh_hist HB words (the tie select's digit width: 12 bits first with 4096, all 10
// bits with 1024).
template <int NT, int CAP, int TIES, int HB>
__device__ void sorted_row(const KernelArgs& a, int64_t row, uint64_t* sh_sort, uint32_t* sh_tk, uint32_t* sh_tp,
                           uint32_t* sh_hist, uint32_t* sh_scan, uint32_t* sh_var) {
  constexpr uint32_t span = (uint32_t)NT * 4u * sort_cv<NT>();
  const int64_t W = a.width;
  const int k = a.k;
  const bool vec = a.vec != 0;
  {
    const int tid = opaque_tid();
    const int32_t sl = (int32_t)uniform((uint32_t)a.seq_lens[row]);
    const uint32_t L = sl < 0 ? 0u : ((int64_t)sl > W ? (uint32_t)W : (uint32_t)sl);
    const uint32_t n = L < (uint32_t)k ? L : (uint32_t)k;
    const uint32_t* m = a.meta + row * kMetaWords;
    const uint32_t prefix = uniform(m[0]);
    const int shift = (int)uniform(m[1]);
    const uint32_t need = uniform(m[2]);
    const uint32_t floor = uniform(m[3]);
    const bool cut = uniform(m[4]) != 0u;
    const float* rowp = a.scores + row * W;
    if (tid < 16) sh_var[tid] = 0;
    for (int i = tid; i < CAP; i += NT) sh_sort[i] = (uint64_t)i;   // unfilled slots: no position, distinct
    __syncthreads();
    if (!cut) {
      const int32_t* sel = a.sel + row * (int64_t)k;
      for (uint32_t j = (uint32_t)tid; j < n; j += NT) {
        const int32_t p = sel[j];
        if (p >= 0 && (uint32_t)p < L) {
          const uint32_t x = order_key_bits(__float_as_uint(rowp[p]));
          sh_sort[j] = ((uint64_t)x << 32) | (uint64_t)(~(uint32_t)p);
        }
      }
      __syncthreads();
    } else {
      // 1. keys above the bin -> sh_sort; the bin's members -> tie list
      for (uint32_t c = 0; c < L; c += span) {
        uint32_t raw[4 * sort_cv<NT>()];
        load_raw<NT, sort_cv<NT>(), kLoadReuse>(raw, rowp, c, L, vec, tid);
#pragma unroll
        for (int j = 0; j < 4 * sort_cv<NT>(); ++j) {
          const uint32_t pos = c + (uint32_t)tid * 4u + (uint32_t)(j >> 2) * (NT * 4) + (uint32_t)(j & 3);
          if (pos >= L) continue;
          const uint32_t x = order_key_bits(raw[j]);
          if (x < floor) continue;
          const uint64_t xp = (uint64_t)x >> shift;
          if (xp > (uint64_t)prefix) {
            const uint32_t s = atomicAdd(&sh_var[0], 1u);
            if (s < (uint32_t)CAP) sh_sort[s] = ((uint64_t)x << 32) | (uint64_t)(~pos);
          } else if (xp == (uint64_t)prefix) {
            const uint32_t t = atomicAdd(&sh_var[1], 1u);
            if (t < (uint32_t)TIES) {
              sh_tk[t] = x;
              sh_tp[t] = pos;
            }
          }
        }
      }
      __syncthreads();
      const uint32_t ngt = uniform(sh_var[0]);
      const uint32_t nties = uniform(sh_var[1]);
      const uint32_t base = ngt < n ? ngt : n;
      const bool in_lds = nties <= (uint32_t)TIES;

      // 2. which bin members: all, or the `need` lowest positions
      uint32_t vprefix = 0;
      int vshift = 32;
      if (nties > need) {
        // MSB-first digits of v: with HB = 4096 bins, 12 + 10 + 10 bits; with
        // HB = 1024 (the small shape, whose histogram is kept small so more
        // workgroups fit a CU), 10 + 10 + 10 + 2 bits
        constexpr int kLevels = HB == kBinsWide ? 3 : 4;
        uint32_t vneed = need;
        for (int level = 0; level < kLevels; ++level) {
          const int dshift = HB == kBinsWide ? (level == 0 ? 20 : (level == 1 ? 10 : 0)) : (level < 3 ? 22 - 10 * level : 0);
          const int width = HB == kBinsWide ? (level == 0 ? 12 : 10) : (level < 3 ? 10 : 2);
          const uint32_t dmask = (1u << width) - 1u;
          const int nb = HB == kBinsWide && level == 0 ? kBinsWide : kBinsNarrow;
          for (int b = tid; b < nb; b += NT) sh_hist[b] = 0;
          __syncthreads();
          if (in_lds) {
            for (uint32_t i = (uint32_t)tid; i < nties; i += NT) {
              const uint32_t v = ~sh_tp[i];
              if (vshift >= 32 || (v >> vshift) == vprefix) atomicAdd(&sh_hist[(v >> dshift) & dmask], 1u);
            }
            __syncthreads();
          } else {
            sorted_tie_pass<NT, CAP>(false, rowp, L, vec, prefix, shift, floor, vprefix, vshift, dshift, dmask, sh_hist,
                                     sh_sort, 0u, sh_var, tid);
          }
          uint32_t bin, gtc, cnt;
          if (nb == kBinsWide) find_threshold<NT, (HB > kBinsNarrow ? HB : kBinsNarrow)>(sh_hist, vneed, sh_scan, sh_var, tid);
          else find_threshold<NT, kBinsNarrow>(sh_hist, vneed, sh_scan, sh_var, tid);
          bin = uniform(sh_var[0]);
          gtc = uniform(sh_var[1]);
          cnt = uniform(sh_var[2]);
          vneed -= gtc;
          vprefix = vshift >= 32 ? bin : ((vprefix << width) | bin);
          vshift = dshift;
          if (cnt == vneed) break;   // positions are distinct: at the last digit the bin holds one
        }
      }

      // 3. the chosen members join sh_sort after the keys above the bin
      if (tid == 0) sh_var[2] = 0;
      __syncthreads();
      if (in_lds) {
        for (uint32_t i = (uint32_t)tid; i < nties; i += NT) {
          const uint32_t v = ~sh_tp[i];
          if (vshift >= 32 || (v >> vshift) >= vprefix) {
            const uint32_t s = base + atomicAdd(&sh_var[2], 1u);
            if (s < (uint32_t)CAP) sh_sort[s] = ((uint64_t)sh_tk[i] << 32) | (uint64_t)v;
          }
        }
        __syncthreads();
      } else {
        sorted_tie_pass<NT, CAP>(true, rowp, L, vec, prefix, shift, floor, vprefix, vshift, 0, 0u, sh_hist, sh_sort, base,
                                 sh_var, tid);
      }

    }


    // 4-5. bitonic sort and output
    bitonic_write<NT>(a, row, n, L, sh_sort, tid);
    __syncthreads();
  }
}

template <int NT, int CAP, int TIES>
__global__ void __launch_bounds__(NT) sorted_rows_kernel(KernelArgs a) {
  __shared__ uint64_t sh_sort[CAP];    // (key << 32) | ~position of the selected
  __shared__ uint32_t sh_tk[TIES];     // threshold-bin members: key
  __shared__ uint32_t sh_tp[TIES];     //                        position
  constexpr int HB = sort_hist_bins<CAP>();
  __shared__ uint32_t sh_hist[HB];
  __shared__ uint32_t sh_scan[64];
  __shared__ uint32_t sh_var[16];
  for (int64_t row = blockIdx.x; row < a.batch; row += gridDim.x)
    sorted_row<NT, CAP, TIES, HB>(a, row, sh_sort, sh_tk, sh_tp, sh_hist, sh_scan, sh_var);
}

// Rank finish: the default sorted finish.  G = a.wgs_per_row workgroups
// share a row (grid = batch x G) and need no synchronisation among them.
// Where the record says the bin was not cut, the selected set is canonical
// and only its order is missing: each workgroup reads all n pairs P =
// (key << 32) | ~position (the keys from the selection launch where it wrote
// them, else gathered from the row) and writes its own n/G of them to their
// slots (rank_pairs_write; a row with a crowded bucket is sorted by its first
// workgroup instead).  Rows whose bin was cut need the row read again: the
// row's first workgroup runs the one-workgroup finish, and the others leave.
template <int NT, int CAP, int TIES, int NB>
__global__ void __launch_bounds__(NT, NT <= 256 ? 8 : 1) sorted_rank_kernel(KernelArgs a) {
  constexpr int HB = sort_hist_bins<CAP>();
  static_assert(NB <= HB && 2 * CAP + NB <= 2 * TIES, "rank finish shape");
  __shared__ uint64_t sh_sort[CAP];
  __shared__ uint32_t sh_t[2 * TIES];   // cut rows: the tie list's keys, then positions
  __shared__ uint32_t sh_hist[HB];
  __shared__ uint32_t sh_scan[64];
  __shared__ uint32_t sh_var[16];
  __shared__ uint64_t sh_mm[2];
  __shared__ uint32_t sh_sub[kSubWords];   // rank_pairs_write's crowded-bucket tables
  __shared__ uint64_t sh_mm2[2];
  // workgroup-major over rows: the rows' first workgroups (which alone finish
  // cut rows) are dispatched first and spread over the XCDs, and when the
  // batch is a multiple of 8 a row's workgroups share one XCD (and its L2,
  // for the gather of the row's keys)
  const int G = a.wgs_per_row;
  const int64_t row = (int64_t)(blockIdx.x % (uint32_t)a.batch);
  const uint32_t g = blockIdx.x / (uint32_t)a.batch;
  if (g >= (uint32_t)G) return;
  const int tid = opaque_tid();
  const int64_t W = a.width;
  const int k = a.k;
  // one round trip: the row's positions and keys (k slots each, in bounds
  // whatever the record says) are requested with the record and the length
  constexpr int kPer = CAP / NT;
  const int32_t* sel = a.sel + row * (int64_t)k;
  const uint32_t* key_row = a.sel_key + row * (int64_t)k;
  int32_t sp[kPer];
  uint32_t sk[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int j = tid + q * NT;
    sp[q] = j < k ? sel[j] : -1;
    sk[q] = j < k ? key_row[j] : 0u;
  }
  const uint32_t rec_cut = a.meta[row * kMetaWords + 4], rec_keys = a.meta[row * kMetaWords + 5];
  const int32_t sl = (int32_t)uniform((uint32_t)a.seq_lens[row]);
  if (uniform(rec_cut) != 0u) {   // cut
    if (g == 0) sorted_row<NT, CAP, TIES, HB>(a, row, sh_sort, sh_t, sh_t + TIES, sh_hist, sh_scan, sh_var);
    return;
  }
  const bool have_keys = uniform(rec_keys) != 0u;
  const uint32_t L = sl < 0 ? 0u : ((int64_t)sl > W ? (uint32_t)W : (uint32_t)sl);
  const uint32_t n = L < (uint32_t)k ? L : (uint32_t)k;
  const float* rowp = a.scores + row * W;
  uint32_t* const sh_cnt = sh_hist;
  pairs_span_init<NT, NB>(sh_cnt, sh_mm, sh_scan, tid);
  __syncthreads();
  uint64_t hi = 0ull, lo = ~0ull;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const uint32_t j = (uint32_t)(tid + q * NT);
    if (j >= n) continue;
    const int32_t p = sp[q];
    // a slot left without a position (none is, for valid input) sorts after every
    // key and is written as -1; j keeps such pairs distinct
    uint64_t P = (uint64_t)j;
    if (p >= 0 && (uint32_t)p < L)
      P = ((uint64_t)(have_keys ? sk[q] : order_key_bits(__float_as_uint(rowp[p]))) << 32) | (uint64_t)(~(uint32_t)p);
    sh_sort[j] = P;
    hi = P > hi ? P : hi;
    lo = P < lo ? P : lo;
  }
  pairs_span(hi, lo, sh_mm, tid);
  const uint32_t j0 = (uint32_t)(((uint64_t)g * n) / (uint32_t)G);
  const uint32_t j1 = (uint32_t)(((uint64_t)(g + 1) * n) / (uint32_t)G);
  if (!rank_pairs_write<NT, NB, CAP>(a, row, n, L, j0, j1, sh_sort, reinterpret_cast<uint64_t*>(sh_t), sh_t + 2 * CAP,
                                sh_cnt, sh_mm, sh_scan, sh_sub, sh_mm2, tid)) {
    // a crowded bucket: the row's first workgroup sorts all n pairs instead
    if (g == 0) {
      for (uint32_t j = n + (uint32_t)tid; j < (uint32_t)CAP; j += NT) sh_sort[j] = (uint64_t)j;
      __syncthreads();
      bitonic_write<NT>(a, row, n, L, sh_sort, tid);
    }
    return;
  }
  if (g == 0) {
    int32_t* o = a.out + row * (int64_t)k;
    int32_t* orw = a.out_raw ? a.out_raw + row * (int64_t)k : nullptr;
    for (int j = (int)n + tid; j < k; j += NT) {
      o[j] = -1;
      if (orw) orw[j] = -1;
    }
  }
}

// Resident workgroups per CU of a kernel's two load forms (the launch picks
// one by the rows' alignment; the host sizes grids for either).
hipError_t occupancy_pair(const void* f_vec, const void* f_scalar, int nt, int* blocks) {
  int b_vec = 0, b_scalar = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&b_vec, f_vec, nt, 0);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&b_scalar, f_scalar, nt, 0);
  *blocks = b_vec < b_scalar ? b_vec : b_scalar;
  return e;
}

// Streaming-kernel shapes: (threads, sample float4 groups per thread, chunk
// float4 groups per thread, chunks in flight, LDS candidates, waves per SIMD,
// page-table row staged in LDS).
#define TOPK_STREAM_VARIANTS(X)      \
  X(0, 1024, 4, 2, 2, 6144, 8, false) \
  X(1, 256, 8, 4, 2, 1920, 4, true)   \
  X(2, 1024, 4, 4, 3, 6144, 4, true)

hipError_t launch_stream_variant(int variant, const KernelArgs& args, hipStream_t stream) {
  switch (variant) {
#define TOPK_LAUNCH_CASE(id, nt, sv, cv, nbuf, cap, waves, ptl)                                                      \
  case id:                                                                                              \
    if (args.vec)                                                                                       \
      hipLaunchKernelGGL((stream_rows_kernel<nt, sv, cv, nbuf, cap, waves, ptl, true>), dim3((unsigned)args.slots), \
                         dim3(nt), 0, stream, args);                                                    \
    else                                                                                                \
      hipLaunchKernelGGL((stream_rows_kernel<nt, sv, cv, nbuf, cap, waves, ptl, false>), dim3((unsigned)args.slots), \
                         dim3(nt), 0, stream, args);                                                    \
    return hipGetLastError();
    TOPK_STREAM_VARIANTS(TOPK_LAUNCH_CASE)
#undef TOPK_LAUNCH_CASE
    default: return hipErrorInvalidValue;
  }
}

hipError_t occupancy_stream_variant(int variant, int* blocks) {
  switch (variant) {
#define TOPK_OCC_CASE(id, nt, sv, cv, nbuf, cap, waves, ptl)                                                         \
  case id:                                                                                              \
    return occupancy_pair(reinterpret_cast<const void*>(&stream_rows_kernel<nt, sv, cv, nbuf, cap, waves, ptl, true>), \
                          reinterpret_cast<const void*>(&stream_rows_kernel<nt, sv, cv, nbuf, cap, waves, ptl, false>), \
                          nt, blocks);
    TOPK_STREAM_VARIANTS(TOPK_OCC_CASE)
#undef TOPK_OCC_CASE
    default: return hipErrorInvalidValue;
  }
}

// Split streaming shapes: (threads, sample float4 groups per thread, chunk
// float4 groups per thread, chunks in flight, LDS candidates, waves per SIMD).
#define TOPK_SPLIT_STREAM_VARIANTS(X) \
  X(0, 1024, 2, 2, 2, 6144, 8, true)   \
  X(1, 1024, 4, 4, 3, 6144, 4, true)

hipError_t launch_split_stream_variant(int variant, const KernelArgs& args, hipStream_t stream) {
  switch (variant) {
#define TOPK_SS_LAUNCH_CASE(id, nt, sv, cv, nbuf, cap, waves, refine)                                            \
  case id:                                                                                                  \
    if (args.meta && args.vec)                                                                              \
      hipLaunchKernelGGL((split_stream_kernel<nt, sv, cv, nbuf, cap, waves, refine, true, true>),           \
                         dim3((unsigned)args.batch * (unsigned)args.wgs_per_row), dim3(nt), 0, stream, args); \
    else if (args.meta)                                                                                     \
      hipLaunchKernelGGL((split_stream_kernel<nt, sv, cv, nbuf, cap, waves, refine, false, true>),          \
                         dim3((unsigned)args.batch * (unsigned)args.wgs_per_row), dim3(nt), 0, stream, args); \
    else if (args.vec)                                                                                      \
      hipLaunchKernelGGL((split_stream_kernel<nt, sv, cv, nbuf, cap, waves, refine, true, false>),          \
                         dim3((unsigned)args.batch * (unsigned)args.wgs_per_row), dim3(nt), 0, stream, args); \
    else                                                                                                    \
      hipLaunchKernelGGL((split_stream_kernel<nt, sv, cv, nbuf, cap, waves, refine, false, false>),         \
                         dim3((unsigned)args.batch * (unsigned)args.wgs_per_row), dim3(nt), 0, stream, args); \
    return hipGetLastError();
    TOPK_SPLIT_STREAM_VARIANTS(TOPK_SS_LAUNCH_CASE)
#undef TOPK_SS_LAUNCH_CASE
    default: return hipErrorInvalidValue;
  }
}

hipError_t occupancy_split_stream_variant(int variant, int* blocks) {
  switch (variant) {
#define TOPK_SS_OCC_CASE(id, nt, sv, cv, nbuf, cap, waves, refine)                                               \
  case id:                                                                                              \
    return occupancy_pair(                                                                               \
        reinterpret_cast<const void*>(&split_stream_kernel<nt, sv, cv, nbuf, cap, waves, refine, true, false>),  \
        reinterpret_cast<const void*>(&split_stream_kernel<nt, sv, cv, nbuf, cap, waves, refine, false, false>), \
        nt, blocks);
    TOPK_SPLIT_STREAM_VARIANTS(TOPK_SS_OCC_CASE)
#undef TOPK_SS_OCC_CASE
    default: return hipErrorInvalidValue;
  }
}

template <int E>
hipError_t launch_e(bool coop, const KernelArgs& args, hipStream_t stream) {
  // Split rows need every workgroup of a row resident at once; the host sizes
  // the grid to at most the device's resident capacity for this kernel, so a
  // regular launch suffices (a cooperative launch would add ~18 us per call).
  const dim3 block(kThreads);
  if (coop) {
    const dim3 grid((unsigned)args.slots * (unsigned)args.wgs_per_row);
    if (args.slots < args.batch)
      hipLaunchKernelGGL((rows_kernel<E, true, true>), grid, block, 0, stream, args);
    else
      hipLaunchKernelGGL((rows_kernel<E, true, false>), grid, block, 0, stream, args);
  } else {
    const dim3 grid((unsigned)args.slots);
    hipLaunchKernelGGL((rows_kernel<E, false, false>), grid, block, 0, stream, args);
  }
  return hipGetLastError();
}

template <int E>
hipError_t occupancy_e(bool coop, int* blocks) {
  if (coop) {
    // the grid is sized once for both split instantiations: the smaller
    // residency holds for either
    int one_pass = 0, cycled = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &one_pass, reinterpret_cast<const void*>(&rows_kernel<E, true, false>), kThreads, 0);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&cycled, reinterpret_cast<const void*>(&rows_kernel<E, true, true>),
                                                       kThreads, 0);
    *blocks = one_pass < cycled ? one_pass : cycled;
    return e;
  }
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, reinterpret_cast<const void*>(&rows_kernel<E, false, false>),
                                                      kThreads, 0);
}

__global__ void __launch_bounds__(256) fill_zero_kernel(uint32_t* p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * 256u + threadIdx.x; i < words; i += (size_t)gridDim.x * 256u) p[i] = 0u;
}

}  // namespace

// The workspace of the entry point that allocates nothing: split-row barrier
// blocks and regions, and the streaming row queue, in the layout of an
// allocated workspace of kScratchSlots slots.  Each device holds its own copy
// for the life of the process.  It is zero-filled once before its first use;
// every kernel leaves it as it found it (zeroes), or, after a wait gave up,
// the launch's last workgroup zeroes it.  Host code must use the address
// scratch_address() returns, never the array's name.
static __device__ __align__(256) uint32_t scratch[kScratchWords];

hipError_t scratch_address(uint32_t** ptr) {
  return hipGetSymbolAddress(reinterpret_cast<void**>(ptr), HIP_SYMBOL(scratch));
}

hipError_t clear_words(uint32_t* p, size_t words, hipStream_t stream) {
  hipLaunchKernelGGL(fill_zero_kernel, dim3(1024), dim3(256), 0, stream, p, words);
  return hipGetLastError();
}

hipError_t launch_rows_pair(const KernelArgs& a, int32_t g16, int32_t slots16, hipStream_t stream) {
  const int64_t n16 = (int64_t)slots16 * g16, n64 = (int64_t)a.slots * a.wgs_per_row;
  hipLaunchKernelGGL(rows_pair_kernel, dim3((unsigned)(n16 > n64 ? n16 : n64)), dim3(kThreads), 0, stream, a, g16,
                     slots16);
  return hipGetLastError();
}

hipError_t rows_pair_occupancy(int* blocks_per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, reinterpret_cast<const void*>(&rows_pair_kernel),
                                                      kThreads, 0);
}

hipError_t launch_rows(int ept_index, bool coop, const KernelArgs& args, hipStream_t stream) {
  switch (ept_index) {
    case 0: return launch_e<4>(coop, args, stream);
    case 1: return launch_e<8>(coop, args, stream);
    case 2: return launch_e<16>(coop, args, stream);
    case 3: return launch_e<32>(coop, args, stream);
    case 4: return launch_e<64>(coop, args, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_stream_rows(int variant, const KernelArgs& args, hipStream_t stream) {
  return launch_stream_variant(variant, args, stream);
}

hipError_t stream_occupancy(int variant, int* blocks_per_cu) { return occupancy_stream_variant(variant, blocks_per_cu); }

hipError_t launch_split_stream(int variant, const KernelArgs& args, hipStream_t stream) {
  return launch_split_stream_variant(variant, args, stream);
}

hipError_t split_stream_occupancy(int variant, int* blocks_per_cu) {
  return occupancy_split_stream_variant(variant, blocks_per_cu);
}

// The sorted finish's two shapes: rows with k <= kSortSmallK take a 256-thread
// workgroup with a 512-entry sort buffer (several rows per CU at once), the
// rest the 1024-thread, 2048-entry one.
hipError_t launch_sorted_rows(const KernelArgs& args, hipStream_t stream) {
  if (args.k <= kSortSmallK)
    hipLaunchKernelGGL((sorted_rows_kernel<kSortSmallThreads, kSortSmallK, 2 * kSortSmallK>), dim3((unsigned)args.slots),
                       dim3(kSortSmallThreads), 0, stream, args);
  else
    hipLaunchKernelGGL((sorted_rows_kernel<kThreads, kMaxK, 2 * kMaxK>), dim3((unsigned)args.slots), dim3(kThreads), 0,
                       stream, args);
  return hipGetLastError();
}

hipError_t launch_sorted_rank(const KernelArgs& args, hipStream_t stream) {
  const unsigned grid = (unsigned)((int64_t)args.batch * args.wgs_per_row);
  if (args.k <= kSortSmallK)
    hipLaunchKernelGGL((sorted_rank_kernel<kSortSmallThreads, kSortSmallK, 2 * kSortSmallK, 1024>), dim3(grid),
                       dim3(kSortSmallThreads), 0, stream, args);
  else
    hipLaunchKernelGGL((sorted_rank_kernel<kThreads, kMaxK, 2 * kMaxK, 4096>), dim3(grid), dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

hipError_t sorted_occupancy(int k, int* blocks_per_cu) {
  if (k <= kSortSmallK)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        blocks_per_cu,
        reinterpret_cast<const void*>(&sorted_rows_kernel<kSortSmallThreads, kSortSmallK, 2 * kSortSmallK>),
        kSortSmallThreads, 0);
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(
      blocks_per_cu, reinterpret_cast<const void*>(&sorted_rows_kernel<kThreads, kMaxK, 2 * kMaxK>), kThreads, 0);
}

int stream_variant_threads(int variant) {
  switch (variant) {
#define TOPK_NT_CASE(id, nt, sv, cv, nbuf, cap, waves, ptl) \
  case id:                                       \
    return nt;
    TOPK_STREAM_VARIANTS(TOPK_NT_CASE)
#undef TOPK_NT_CASE
    default: return 0;
  }
}

hipError_t rows_occupancy(int ept_index, bool coop, int* blocks_per_cu) {
  switch (ept_index) {
    case 0: return occupancy_e<4>(coop, blocks_per_cu);
    case 1: return occupancy_e<8>(coop, blocks_per_cu);
    case 2: return occupancy_e<16>(coop, blocks_per_cu);
    case 3: return occupancy_e<32>(coop, blocks_per_cu);
    case 4: return occupancy_e<64>(coop, blocks_per_cu);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace topk
