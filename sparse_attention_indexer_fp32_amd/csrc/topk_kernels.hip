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
//   * Selected positions go to a staging list (LDS, or global when the row is
//     split); after a barrier one pass gathers the page-table entries and
//     writes out_idx / out_raw coalesced, -1 padded.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "topk_internal.h"

namespace topk {
namespace {

constexpr uint32_t kSpinLimit = 1u << 21;   // bounded wait: ~seconds, then flag a fault and go on

enum Mode : int { kModeNone = 0, kModeTakeAll = 1, kModeTies = 2, kModeCands = 3 };

// fp32 -> uint32 whose unsigned order is the value order (-0.0 just below +0.0).
// Key 0 belongs only to the NaN pattern 0xFFFFFFFF, so 0 marks "no element".
__device__ __forceinline__ uint32_t order_key_bits(uint32_t u) {
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Word 3 of a CDNA (gfx9-family) raw buffer descriptor: 32-bit data format,
// no swizzle; loads past num_records return zero.
constexpr int kBufferWord3 = 0x00020000;

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

// ---- agent-scope (whole-GPU, across XCDs) memory operations ----------------
__device__ __forceinline__ void g_add(uint32_t* p, uint32_t v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t g_add_ret(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t g_load(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void g_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- scans -----------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v, int tid) {
  const int lane = tid & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// Exclusive scan over the workgroup in thread order; `total` gets the sum.
// sh_scan needs kWaves + 1 words.  Contains barriers: call uniformly.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* sh_scan, uint32_t& total,
                                                        int tid) {
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const uint32_t inc = wave_inclusive_scan(v, tid);
  if (lane == 63) sh_scan[wid] = inc;
  __syncthreads();
  if (wid == 0) {
    const uint32_t w = lane < kWaves ? sh_scan[lane] : 0u;
    const uint32_t wi = wave_inclusive_scan(w, tid);
    if (lane < kWaves) sh_scan[lane] = wi - w;
    if (lane == kWaves - 1) sh_scan[kWaves] = wi;
  }
  __syncthreads();
  const uint32_t r = sh_scan[wid] + inc - v;
  total = sh_scan[kWaves];
  __syncthreads();
  return r;
}

// Threshold bin of histogram h[0, nb): the highest bin t with
// sum_{b >= t} h[b] >= need.  Writes sh_var[0] = t, sh_var[1] = count in bins
// above t, sh_var[2] = h[t].  (If the histogram holds fewer than `need`
// elements -- impossible for valid input -- it reports bin 0 with counts 0.)
__device__ __forceinline__ void find_threshold(const uint32_t* h, int nb, uint32_t need, uint32_t* sh_scan,
                                               uint32_t* sh_var, int tid) {
  const int per = nb / kThreads;
  const int top = nb - per * tid;   // this thread covers bins [top - per, top), highest first
  uint32_t s = 0;
  for (int i = 1; i <= per; ++i) s += h[top - i];
  if (tid == 0) {
    sh_var[0] = 0;
    sh_var[1] = 0;
    sh_var[2] = 0;
  }
  uint32_t total;
  const uint32_t before = block_exclusive_scan(s, sh_scan, total, tid);
  if (before < need && before + s >= need) {
    uint32_t acc = before;
    for (int i = 1; i <= per; ++i) {
      const uint32_t c = h[top - i];
      if (acc + c >= need) {
        sh_var[0] = (uint32_t)(top - i);
        sh_var[1] = acc;
        sh_var[2] = c;
        break;
      }
      acc += c;
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
// the device's resident-workgroup capacity, so all G are running.  Sense is a
// generation counter: the last arriver resets the arrival count (drained
// before it bumps the generation), so the barrier resets itself across calls
// and graph replays.  The wait is bounded: on timeout the fault word is set
// and every later wait returns at once, so the kernel always drains.
__device__ __forceinline__ void row_barrier(uint32_t* bar, int G, uint32_t* fault, int tid) {
  wave_mem_drain();
  __syncthreads();
  if (tid == 0) {
    const uint32_t gen = g_load(bar + 1);
    wave_mem_drain();   // the generation is read before this workgroup's arrival
    const uint32_t old = g_add_ret(bar, 1u);
    if (old == (uint32_t)G - 1) {
      g_store(bar, 0u);
      wave_mem_drain();
      g_add(bar + 1, 1u);
    } else if (g_load(fault) == 0u) {
      uint32_t spins = 0;
      while (g_load(bar + 1) == gen) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kSpinLimit) {
          g_store(fault, 1u);
          break;
        }
      }
    }
    wave_mem_drain();
  }
  __syncthreads();
}

// Gather + transform pass: slot j < n holds raw position r (trivial rows: r = j);
// out = page_table[row, r >> log2_page] << log2_page | (r & (page_size - 1)).
// Slots past n, and any r outside [0, L), give -1.
__device__ __forceinline__ void write_row_output(const KernelArgs& a, int64_t row, int64_t L, int n, bool trivial,
                                                 const int32_t* sh_raw, int tid) {
  const int k = a.k;
  const int s = a.log2_page;
  const uint32_t pmask = (1u << s) - 1u;
  int32_t* o = a.out + row * (int64_t)k;
  int32_t* orw = a.out_raw ? a.out_raw + row * (int64_t)k : nullptr;
  const int32_t* pt = a.page_table + row * a.pages_per_row;
  for (int j = tid; j < k; j += kThreads) {
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
__device__ __forceinline__ void hist_pass0(const uint32_t (&key)[E], uint32_t need, uint32_t* h,
                                           uint32_t* sh_scan, uint32_t* sh_var, int tid) {
  constexpr int S = SampleSlots<E>::value;
#pragma unroll
  for (int j = 0; j < S; ++j)
    if (key[j]) atomicAdd(&h[key[j] >> 20], 1u);
  if (S == E) return;
  __syncthreads();
  find_threshold(h, kBinsWide, need, sh_scan, sh_var, tid);
  // Bin >= 1 also excludes key 0 (no element).
  const uint32_t gate = uniform(sh_var[0]) > 1u ? uniform(sh_var[0]) : 1u;
#pragma unroll
  for (int j = S; j < E; ++j)
    if ((key[j] >> 20) >= gate) atomicAdd(&h[key[j] >> 20], 1u);
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

// Finishes a row from its threshold-bin candidates held in LDS: the remaining
// radix digits, then the compaction into staging slots [base, base + need).
__device__ __forceinline__ void finish_candidates(int ncand, int pass_done, uint32_t prefix, int shift, uint32_t need,
                                  uint32_t base, uint32_t* sh_hist, const uint32_t* sh_ckey,
                                                  const int32_t* sh_cpos, int32_t* sh_raw, uint32_t* sh_scan,
                                                  uint32_t* sh_var, int tid) {
  const uint32_t need0 = need;
  int mode = kModeTies;
  for (int pass = pass_done + 1; pass < 3; ++pass) {
    for (int b = tid; b < kBinsNarrow; b += kThreads) sh_hist[b] = 0;
    __syncthreads();
    for (int i = tid; i < ncand; i += kThreads) {
      const uint32_t x = sh_ckey[i];
      if ((x >> shift) == prefix) atomicAdd(&sh_hist[(x >> (shift - 10)) & 1023u], 1u);
    }
    __syncthreads();
    find_threshold(sh_hist, kBinsNarrow, need, sh_scan, sh_var, tid);
    const uint32_t bin = uniform(sh_var[0]), gt = uniform(sh_var[1]), cnt = uniform(sh_var[2]);
    need -= gt;
    prefix = (prefix << 10) | bin;
    shift -= 10;
    if (cnt == need) {
      mode = kModeTakeAll;
      break;
    }
  }
  (void)mode;  // with shift == 0 the equal keys are identical: any `need` of them
  if (tid == 0) {
    sh_var[8] = 0;
    sh_var[9] = 0;
  }
  __syncthreads();
  const uint32_t gbase = base, ebase = base + (need0 - need);
  for (int i = tid; i < ncand; i += kThreads) {
    const uint32_t x = sh_ckey[i] >> shift;
    if (x > prefix) {
      const uint32_t s = atomicAdd(&sh_var[8], 1u);
      if (gbase + s < ebase && gbase + s < (uint32_t)kMaxK) sh_raw[gbase + s] = sh_cpos[i];
    } else if (x == prefix) {
      const uint32_t e = atomicAdd(&sh_var[9], 1u);
      if (e < need && ebase + e < (uint32_t)kMaxK) sh_raw[ebase + e] = sh_cpos[i];
    }
  }
  __syncthreads();
}

template <int E, bool COOP>
__global__ void __launch_bounds__(kThreads) rows_kernel(KernelArgs a) {
  __shared__ uint32_t sh_hist[kBinsWide];
  __shared__ int32_t sh_raw[kMaxK + 64];   // + one trash word per lane
  __shared__ uint32_t sh_scan[kWaves + 1];
  __shared__ uint32_t sh_var[16];
  __shared__ uint32_t sh_ckey[COOP ? kCandCap : 1];
  __shared__ int32_t sh_cpos[COOP ? kCandCap : 1];

  const int G = COOP ? a.wgs_per_row : 1;
  const int slot = (int)blockIdx.x / G;
  const int g = (int)blockIdx.x - slot * G;
  const int64_t C = (int64_t)kThreads * E;
  const int64_t W = a.width;
  const int k = a.k;
  uint32_t* fault = a.ws;
  uint32_t* bar = COOP ? a.ws + kHdrWords + (size_t)slot * kBarWords : nullptr;

  int nsplit = 0;   // split rows this slot has finished: picks the workspace region parity
  for (int it = 0;; ++it) {
    const int tid = opaque_tid();
    const int64_t row = (int64_t)slot + (int64_t)it * a.slots;
    if (row >= a.batch) break;
    const int32_t sl = (int32_t)uniform((uint32_t)a.seq_lens[row]);
    const int64_t L = sl < 0 ? 0 : ((int64_t)sl > W ? W : (int64_t)sl);
    const int n = L < (int64_t)k ? (int)L : k;
    if (L <= (int64_t)k) {  // every valid position is selected (uniform over the row's workgroups)
      if (g == 0) write_row_output(a, row, L, n, true, sh_raw, tid);
      continue;
    }
    constexpr bool split = COOP;   // the host launches the split kernel only with G > 1
    // Consecutive split rows of a slot alternate regions.  A region is reused
    // two split rows later, after every workgroup of the slot has passed the
    // in-between row's first barrier -- which the finisher that clears it
    // reaches only after clearing.
    uint32_t* region = split ? a.ws + kHdrWords + (size_t)a.ws_slots * kBarWords +
                                   ((size_t)slot * 2 + (size_t)(nsplit & 1)) * kRegionWords
                             : nullptr;
    nsplit += split ? 1 : 0;

    for (int j = tid; j < k; j += kThreads) sh_raw[j] = -1;

    // ---- load this workgroup's share of the row into registers (one HBM read)
    const float* rowp = a.scores + row * W;
    // Element j of thread tid sits at position c0 + 4*tid + 4096*(j/4) + j%4:
    // each group of four is one dwordx4 buffer load when the row is 16-byte
    // aligned, else four dword loads of the same positions.  The buffer
    // descriptor covers only the valid part of this chunk, so the hardware
    // bounds check returns 0 past seq_len (and past the tensor) without a
    // branch; those slots become key 0 ("no element").  All loads are issued
    // before the first one is consumed.
    const uint32_t c0 = (uint32_t)g * (uint32_t)C;
    const int64_t rem = L - (int64_t)c0;
    const uint32_t nvalid = rem <= 0 ? 0u : (rem >= C ? (uint32_t)C : (uint32_t)rem);
    const uint32_t pbase = c0 + (uint32_t)tid * 4u;
    uint32_t key[E];
    {
      // With dwordx4 loads the descriptor spans whole 16-byte groups (still
      // inside the row: the width is a multiple of 4 then), so no load
      // straddles num_records; positions past seq_len are masked below.
      const uint32_t nbytes = a.vec ? ((nvalid + 3u) & ~3u) * 4u : nvalid * 4u;
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(rowp) + c0, (short)0, (int)nbytes, kBufferWord3);
      const uint32_t voff = (uint32_t)tid * 16u;
      const uint32_t lpos = (uint32_t)tid * 4u;   // position within the chunk
      if (a.vec) {
#pragma unroll
        for (int v = 0; v < E / 4; ++v) {
          const auto x = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, v * (kThreads * 16), 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // valid iff lpos + offset < nvalid; the limit is a scalar
            const int32_t lim = (int32_t)nvalid - (v * kThreads * 4 + i);
            key[4 * v + i] = ((int32_t)lpos < lim) ? order_key_bits(x[i]) : 0u;
          }
        }
      } else {
#pragma unroll
        for (int v = 0; v < E / 4; ++v) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t x = __builtin_amdgcn_raw_buffer_load_b32(rsrc, voff, v * (kThreads * 16) + 4 * i, 0);
            const int32_t lim = (int32_t)nvalid - (v * kThreads * 4 + i);
            key[4 * v + i] = ((int32_t)lpos < lim) ? order_key_bits(x) : 0u;
          }
        }
      }
    }
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
      if (pass == 0) hist_pass0<E>(key, need, sh_hist, sh_scan, sh_var, tid);
      else hist_resident<E>(key, pass, prefix, sh_hist);
      __syncthreads();
      if (split) {
        uint32_t* gh = region + (pass == 0 ? kRegHist0 : pass == 1 ? kRegHist1 : kRegHist2);
        for (int b = tid; b < nb; b += kThreads) {
          const uint32_t c = sh_hist[b];
          if (c) g_add(gh + b, c);
        }
        row_barrier(bar, G, fault, tid);
        for (int b = tid; b < nb; b += kThreads) sh_hist[b] = g_load(gh + b);
        __syncthreads();
      }
      find_threshold(sh_hist, nb, need, sh_scan, sh_var, tid);
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
    const uint32_t off = block_exclusive_scan((cg << 17) | ce, sh_scan, tot, tid);
    uint32_t off_g = off >> 17, off_e = off & 0x1FFFFu;
    if (split) {
      if (tid == 0) {
        const uint32_t tg = tot >> 17, te = tot & 0x1FFFFu;
        sh_var[4] = tg ? g_add_ret(region + kRegCtr + kCtrGreater, tg) : 0u;
        sh_var[5] = te ? g_add_ret(region + kRegCtr + kCtrEqual, te) : 0u;
      }
      __syncthreads();
      off_g += uniform(sh_var[4]);
      off_e += uniform(sh_var[5]);
    }
    // Selected keys are rare: a wave skips a register slot unless one of its
    // lanes holds a key at or above the threshold prefix.  Inside, lanes that
    // have nothing to store write a private trash word instead of branching.
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
      } else if (mode == kModeCands) {
        if (isg && sg < n_gt) g_store(region + kRegRaw + sg, (uint32_t)pos_of(j));
        if (ise && se < (uint32_t)kCandCap) {
          g_store(region + kRegCandKey + se, x);
          g_store(region + kRegCandPos + se, (uint32_t)pos_of(j));
        }
      } else {
        const uint32_t slot = (isg && sg < n_gt) ? sg : ((ise && se < need) ? n_gt + se : 0xFFFFFFFFu);
        if (slot != 0xFFFFFFFFu) g_store(region + kRegRaw + slot, (uint32_t)pos_of(j));
      }
    }

    if (!split) {
      __syncthreads();
      write_row_output(a, row, L, n, false, sh_raw, tid);
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

    const uint32_t filled = mode == kModeCands ? n_gt : (uint32_t)n;
    for (uint32_t j = tid; j < filled; j += kThreads) sh_raw[j] = (int32_t)g_load(region + kRegRaw + j);
    if (mode == kModeCands) {
      const int ncand = (int)(cnt < (uint32_t)kCandCap ? cnt : (uint32_t)kCandCap);
      for (int i = tid; i < ncand; i += kThreads) {
        sh_ckey[i] = g_load(region + kRegCandKey + i);
        sh_cpos[i] = (int32_t)g_load(region + kRegCandPos + i);
      }
      __syncthreads();
      finish_candidates(ncand, pass, prefix, shift, need, n_gt, sh_hist, sh_ckey, sh_cpos, sh_raw, sh_scan,
                        sh_var, tid);
    }
    __syncthreads();
    write_row_output(a, row, L, n, false, sh_raw, tid);
    // leave the region zeroed for the row this slot handles two iterations on
    for (int b = tid; b < kBinsWide; b += kThreads) g_store(region + kRegHist0 + b, 0u);
    for (int b = tid; b < kBinsNarrow; b += kThreads) {
      g_store(region + kRegHist1 + b, 0u);
      g_store(region + kRegHist2 + b, 0u);
    }
    if (tid < 64) g_store(region + kRegCtr + tid, 0u);
    __syncthreads();
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
    hipLaunchKernelGGL((rows_kernel<E, true>), grid, block, 0, stream, args);
  } else {
    const dim3 grid((unsigned)args.slots);
    hipLaunchKernelGGL((rows_kernel<E, false>), grid, block, 0, stream, args);
  }
  return hipGetLastError();
}

template <int E>
hipError_t occupancy_e(bool coop, int* blocks) {
  if (coop)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, reinterpret_cast<const void*>(&rows_kernel<E, true>),
                                                        kThreads, 0);
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, reinterpret_cast<const void*>(&rows_kernel<E, false>),
                                                      kThreads, 0);
}

}  // namespace

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
