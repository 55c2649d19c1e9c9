// Indexer scoring on gfx950: the step before the top-k (LiteTopk PR #32094
// "Add LiteTopk fused indexer top-k prefill path for SM100": Summary and the
// Background list; the Validation section's reference formula).
//
//   score[r, j] = s[j] * sum_h w[r, h] * relu(q[r, h, :] . kv[j, :]),
//   j in row r's key range [ks[r], ke[r]), H = 32 heads of D = 128 (GLM shape).
//
// Two kernels share one scoring routine, so they produce the same fp32 value
// for every (row, position):
//   * logits_kernel<false> writes the scores densely (row-relative columns):
//     the dense path whose [rows, length] buffer the fused path avoids;
//   * logits_kernel<true> is the fused scan: each wave keeps, per row, a
//     compact candidate list in global memory behind a gate that only
//     tightens, and the lists are then reduced by the exact top-k.
//
// Matrix cores.  q and kv arrive as fp8 E4M3 codes.  gfx950's fp8 matrix
// instructions sum their products with less than fp32 precision (measured:
// up to ~2^-12 of the sum of |products| on wide-range inputs), while every
// E4M3 value is exact in bf16 and the bf16 instruction sums like fp32.  So
// both operands are widened to bf16 (hardware conversion, exact) and the
// contraction runs on v_mfma_f32_32x32x16_bf16: M = the 32 heads of one query
// row, N = 32 key positions, K = 128 in eight steps.  That gives a score
// within a few fp32 rounding errors of the exact value, at half the fp8 peak.
//
// Tiling.  A workgroup of 4 waves owns 8 query rows (2 per wave, their q held
// in registers as bf16) and a window of key positions.  Key stages of 64
// positions (two 32-position tiles) are loaded once per workgroup (32 bytes
// per thread, two stages ahead), widened to bf16 into LDS (double-buffered,
// 16-byte chunks XOR-swizzled by position so the 32 positions a half-wave
// reads fall in different banks), and read by all four waves.  The epilogue (relu, head weights, the partner half-wave's
// 16 heads, the position's scale) runs on the accumulator registers.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "indexer_internal.h"

namespace indexer {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kHeads = 32;
constexpr int kDim = 128;
constexpr int kTile = 32;             // key positions per tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 2;
constexpr int kRowsPerWg = kWaves * kRowsPerWave;
constexpr int kTileBytesBf16 = kTile * kDim * 2;   // 8 KB
constexpr int kHistBins = 2048;

// order key of an fp32 value: unsigned order == value order (-0 below +0)
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Eight fp8 codes (two dwords) -> eight bf16 values, exact.
__device__ __forceinline__ bf16x8 widen8(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// LDS byte offset of 16-byte chunk c (0..15) of position n's bf16 row.
__device__ __forceinline__ int tile_offset(int n, int c) { return n * (kDim * 2) + ((c ^ (n & 15)) << 4); }

// A lane's view of one query row: head h = lane % 32 and the half hb = lane / 32
// of the head dimension it feeds, as bf16, ready for the eight K steps; and
// the 16 head weights its accumulator rows carry.
struct RowOperand {
  bf16x8 a[8];
  float w[16];
};

// Step s of the contraction pairs, on both operands, the 8 values
// d = hb * 64 + s * 8 + (0..7) of the lane's half: every d in [0, 128) is used
// exactly once, and A and B agree on which d sits in which slot.
__device__ __forceinline__ void load_row(const uint8_t* q, const float* weights, int64_t row, bool live, int lane,
                                         RowOperand& op) {
  const int h = lane & 31, hb = lane >> 5;
  if (live) {
    const uint4* src = reinterpret_cast<const uint4*>(q + (row * kHeads + h) * kDim + hb * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = src[i];
      op.a[2 * i] = widen8(v.x, v.y);
      op.a[2 * i + 1] = widen8(v.z, v.w);
    }
    // accumulator register r of this lane holds head (r / 4) * 8 + hb * 4 + r % 4
#pragma unroll
    for (int r = 0; r < 16; ++r) op.w[r] = weights[row * kHeads + (r >> 2) * 8 + hb * 4 + (r & 3)];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) op.a[i] = bf16x8{};
#pragma unroll
    for (int r = 0; r < 16; ++r) op.w[r] = 0.f;
  }
}

// Epilogue of one query row against a tile: relu of each head's dot
// product, the head weights, the partner half-wave's 16 heads, the position's
// scale.  Every lane returns the score of position n = lane % 32 of the tile
// (both half-waves hold it).  The order of the operations is fixed, so every
// kernel that calls this gets the same fp32 value.
//
// relu is a signed-integer max of the value's bits with 0: negative floats
// (and -0) have negative bit patterns and become +0, the rest pass unchanged.
// That is max(x, 0) for every non-NaN x in one instruction (a float max of an
// accumulator costs a quieting max first); a -0 from the float form could not
// change the sum either, which starts at +0.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

__device__ __forceinline__ float finish_score(const RowOperand& op, const f32x16& acc, float scale, int lane) {
  float part = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) part = fmaf(op.w[r], relu(acc[r]), part);
  // The other 16 heads of the same position sit in lane ^ 32.  The swap
  // exchanges the upper half-wave of its first operand with the lower
  // half-wave of its second: with both = part, lane l < 32 finds lane l + 32
  // in the second result and lane l >= 32 finds lane l - 32 in the first.
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
  const float other = __uint_as_float(lane < 32 ? sw[1] : sw[0]);
  return (part + other) * scale;
}

struct RowRange {
  int64_t lo, hi;   // [lo, hi) of key positions, clamped; hi <= lo when empty
};

__device__ __forceinline__ RowRange row_range(const ScanArgs& a, int64_t row) {
  RowRange r{0, 0};
  if (row < a.num_q) {
    int64_t lo = a.ks[row], hi = a.ke[row];
    lo = lo < 0 ? 0 : (lo > a.num_kv ? a.num_kv : lo);
    hi = hi < 0 ? 0 : (hi > a.num_kv ? a.num_kv : hi);
    r.lo = lo;
    r.hi = hi;
  }
  return r;
}

// ---- candidate lists (fused scan) -------------------------------------------------------------
//
// Row r's list in window w holds (score, position) pairs at
// cand_score / cand_pos + ((r * nwin + w) * cap).  The gate is an order key;
// positions whose key is >= gate are appended.  Invariant: for every position
// of the window seen so far that is not in the list, the list holds at least
// k entries whose keys are >= its key -- so the list's top-k is a top-k of
// everything seen (LiteTopk PR #32094: the threshold only tightens, stays at or
// below the true k-th best, and a stale gate admits extras but drops nothing).

__device__ __forceinline__ int wave_prefix(uint64_t mask, int lane) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// Wave-level: the bin t of hist[0..bins) (bins a multiple of 64) with
// count(bins > t) < need <= count(bins >= t).  Returns t; *above = count(> t),
// *in_bin = hist[t].  Requires sum(hist) >= need >= 1.
__device__ int find_bin(const uint32_t* hist, int bins, uint32_t need, int lane, uint32_t* above, uint32_t* in_bin) {
  const int per = bins / 64;
  uint32_t own = 0;
  for (int i = 0; i < per; ++i) own += hist[lane * per + i];
  // exclusive suffix sum over lanes (lanes above this one)
  uint32_t incl = own;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t v = __shfl_down(incl, d);
    if (lane + d < 64) incl += v;
  }
  const uint32_t excl = incl - own;
  const bool mine = excl < need && need <= incl;
  const uint64_t m = __ballot(mine);
  const int src = (int)__builtin_ctzll(m);   // exactly one lane
  uint32_t t = 0, ab = 0, ib = 0;
  if (lane == src) {
    uint32_t acc = excl;
    for (int i = per - 1; i >= 0; --i) {
      const uint32_t c = hist[lane * per + i];
      if (acc + c >= need) {
        t = (uint32_t)(lane * per + i);
        ab = acc;
        ib = c;
        break;
      }
      acc += c;
    }
  }
  *above = (uint32_t)__shfl((int)ab, src);
  *in_bin = (uint32_t)__shfl((int)ib, src);
  return __shfl((int)t, src);
}

__device__ __forceinline__ void clear_hist(uint32_t* hist, int bins, int lane) {
  for (int i = lane; i < bins; i += 64) hist[i] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Histogram of the keys in the list that match `prefix` above bit `lo_bit + width`.
// The list passes keep kListBatch loads per lane in flight: the list was just
// written and its reads come from L2, so one load at a time would make a trim
// a chain of memory latencies while the workgroup's other waves wait.
constexpr int kListBatch = 16;

// Gate bins: per (wave, row), kGateBins counters over [lo, lo + kGateBins << shift)
// of the order key, the last one also counting every key above.  A trim sets
// lo = the new gate, fits shift so the bins reach the kept list's
// (need/4)-th largest key, and counts the kept entries; the list writes count
// the new ones.  The gate may then rise to the highest bin edge with `need`
// list entries at or above it: every position it skips has `need` entries at
// least as large.  shift = 32 marks the bins as unset (before a first trim).
constexpr int kGateBins = 48;

__device__ __forceinline__ uint32_t gate_bin(uint32_t key, uint32_t lo, uint32_t shift) {
  const uint64_t b = (uint64_t)(key - lo) >> shift;
  return b < (uint64_t)(kGateBins - 1) ? (uint32_t)b : (uint32_t)(kGateBins - 1);
}

__device__ void list_hist(const float* sc, int count, uint32_t* hist, int lane, int shift, uint32_t mask,
                          int match_shift, uint32_t match) {
  clear_hist(hist, (int)mask + 1 < 64 ? 64 : (int)mask + 1, lane);
  for (int base = 0; base < count; base += 64 * kListBatch) {
    float v[kListBatch];
#pragma unroll
    for (int b = 0; b < kListBatch; ++b) {
      const int i = base + b * 64 + lane;
      v[b] = i < count ? sc[i] : 0.f;
    }
#pragma unroll
    for (int b = 0; b < kListBatch; ++b) {
      const int i = base + b * 64 + lane;
      const uint32_t key = order_key(v[b]);
      if (i < count && (match_shift >= 32 || (key >> match_shift) == match))
        atomicAdd(&hist[(key >> shift) & mask], 1u);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Shrinks a list of `count` > need entries.  Exact mode keeps every entry
// whose key is above the need-th largest key T and the first (in list order)
// of those equal to T, need entries in all, and sets gate = T + 1.  Otherwise,
// when the 11-bit (else the 22-bit) key prefix bin holding the need-th key
// leaves at most `room` entries at or above its lower edge, it keeps those
// and sets gate = that edge.  Returns the new count and gate by value: a gate
// passed by address would keep the caller's gate in scratch memory, and every
// gate test would then reload it and wait on the load counter, i.e. on the
// key stages still in flight.  The list's earlier stores of this wave are
// made visible to its loads first.
// The gate returned is at least cur_gate (a valid gate stays valid: the
// trim keeps every entry at or above it that the k-th largest key needs).
// With gbins, the gate bins are refitted to the kept list (see kGateBins).
struct Trimmed {
  int count;
  uint32_t gate;
  uint32_t bins_lo, bins_shift;
};

__device__ __attribute__((noinline)) Trimmed compact_list(float* sc, int32_t* ps, int count, uint32_t need, int room,
                                                          bool exact_only, uint32_t* hist, int lane, uint32_t cur_gate,
                                                          uint32_t* gbins) {
  __threadfence();
  uint32_t above = 0, in_bin = 0;
  list_hist(sc, count, hist, lane, 21, 0x7FF, 32, 0);
  const uint32_t t1 = (uint32_t)find_bin(hist, 2048, need, lane, &above, &in_bin);
  uint64_t bins_top = 0;   // above the kept list's (need/4)-th largest key
  if (gbins != nullptr) {
    uint32_t aq = 0, iq = 0;
    const uint32_t tq = (uint32_t)find_bin(hist, 2048, need / 4 > 0 ? need / 4 : 1, lane, &aq, &iq);
    bins_top = ((uint64_t)tq + 1) << 21;
  }
  uint32_t lo_key;   // keep keys >= lo_key (all) ...
  uint32_t eq_key = 0;   // ... except that only the first `eq_need` equal to eq_key are kept
  uint32_t eq_need = 0xFFFFFFFFu;
  uint32_t new_gate;
  if (!exact_only && above + in_bin <= (uint32_t)room) {
    lo_key = t1 << 21;
    new_gate = lo_key;
  } else {
    uint32_t above2 = 0, in2 = 0, above3 = 0, in3 = 0;
    list_hist(sc, count, hist, lane, 10, 0x7FF, 21, t1);
    const uint32_t t2 = (uint32_t)find_bin(hist, 2048, need - above, lane, &above2, &in2);
    const uint32_t p2 = (t1 << 11) | t2;
    if (!exact_only && above + above2 + in2 <= (uint32_t)room) {
      // the 22-bit bin's lower edge already leaves at most `room` entries
      lo_key = p2 << 10;
      new_gate = lo_key;
    } else {
      list_hist(sc, count, hist, lane, 0, 0x3FF, 10, p2);
      const uint32_t t3 = (uint32_t)find_bin(hist, 1024, need - above - above2, lane, &above3, &in3);
      const uint32_t T = (p2 << 10) | t3;
      lo_key = T;
      eq_key = T;
      eq_need = need - above - above2 - above3;
      new_gate = T == 0xFFFFFFFFu ? T : T + 1;
    }
  }
  if (new_gate < cur_gate) new_gate = cur_gate;
  uint32_t bins_lo = 0, bins_shift = 32;
  if (gbins != nullptr) {
    bins_lo = new_gate;
    const uint64_t span = bins_top > bins_lo ? bins_top - bins_lo : 1;
    bins_shift = 0;
    while (((uint64_t)kGateBins << bins_shift) < span) ++bins_shift;
    if (lane < kGateBins) gbins[lane] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
  // In place and order-preserving.  A batch is loaded before any of it is
  // written, and the entries of element b of a batch go to indices below
  // base + (b + 1) * 64, under every index a later element or batch reads.
  int out = 0;
  uint32_t eq_seen = 0;
  const bool cut = eq_need != 0xFFFFFFFFu;
  for (int base = 0; base < count; base += 64 * kListBatch) {
    float sv[kListBatch];
    int32_t pv[kListBatch];
#pragma unroll
    for (int b = 0; b < kListBatch; ++b) {
      const int i = base + b * 64 + lane;
      sv[b] = i < count ? sc[i] : 0.f;
      pv[b] = i < count ? ps[i] : 0;
    }
#pragma unroll
    for (int b = 0; b < kListBatch; ++b) {
      const int i = base + b * 64 + lane;
      const uint32_t key = order_key(sv[b]);
      const bool eq = cut && i < count && key == eq_key;
      const uint64_t eqm = __ballot(eq);
      const uint32_t eq_rank = eq_seen + (uint32_t)wave_prefix(eqm, lane);
      eq_seen += (uint32_t)__builtin_popcountll(eqm);
      const bool keep = i < count && key >= lo_key && (!eq || eq_rank < eq_need);
      const uint64_t km = __ballot(keep);
      if (keep) {
        const int o = out + wave_prefix(km, lane);
        sc[o] = sv[b];
        ps[o] = pv[b];
        if (gbins != nullptr && key >= bins_lo) atomicAdd(&gbins[gate_bin(key, bins_lo, bins_shift)], 1u);
      }
      out += __builtin_popcountll(km);
    }
  }
  return Trimmed{out, new_gate, bins_lo, bins_shift};
}

// Counts `n` newly written list entries (their scores in `app`) into a row's
// gate bins (lo = par[0], shift = par[1], set), then returns the highest bin
// edge with `need` list entries at or above it if it is above `gate`, else
// `gate`.  Not inlined: it runs only on list writes after a first trim, and
// inline it would crowd the scoring loop's registers.
__device__ __attribute__((noinline)) uint32_t raise_gate(const float* app, int n, uint32_t* gbins, const uint32_t* par,
                                                         uint32_t need, uint32_t gate, int lane) {
  const uint32_t lo = par[0], shift = par[1];
  for (int e = lane; e < n; e += 64) {
    const uint32_t key = order_key(app[e]);
    if (key >= lo) atomicAdd(&gbins[gate_bin(key, lo, shift)], 1u);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  uint32_t c = lane < kGateBins ? gbins[lane] : 0u;   // then: count of bins >= lane
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t up = __shfl_down(c, d);
    if (lane + d < 64) c += up;
  }
  const uint64_t m = __ballot(lane < kGateBins && c >= need);
  if (m != 0) {
    const uint64_t edge = (uint64_t)lo + ((uint64_t)(63 - __builtin_clzll(m)) << shift);
    if (edge <= 0xFFFFFFFFull && (uint32_t)edge > gate) return (uint32_t)edge;
  }
  return gate;
}

}  // namespace

// Key positions staged per barrier: two 32-position MFMA tiles.
constexpr int kStage = 2 * kTile;
constexpr int kStageBytesBf16 = kStage * kDim * 2;   // 16 KB
// Appends held in LDS per (wave, row) before they go to the global list:
// room for two stages' worth beyond the stage being computed.
constexpr int kAppendCap = 3 * kStage;

// Calibrated start (fused scan).  Before its scan, a workgroup scores
// kCalStages stages spread evenly over its span (every position appended),
// and each row starts its scan behind the gate at rank m of that sample: the
// sample holds on average mu = n S / L of the row's n best positions (S of its
// L positions sampled), and m = mu + 7 sqrt(mu) + 6.  The scan then starts
// from an empty list.  Every list entry is at or above the starting gate, so a
// row that ends with at least n entries has a top-n in its list (a position
// skipped below the starting gate is below all of them; one skipped after a
// trim is covered by the trim's k entries); a row that ends with fewer is
// scanned again from gate 0.  This is the page's prefix calibration of the
// initial threshold, taken from samples of the whole window so that it does
// not depend on where in the row the best positions lie, and made safe by the
// end-of-scan count rather than by the sample's statistics.
constexpr int kCalStages = 32;

__device__ __forceinline__ int calibration_rank(int64_t n, int64_t sampled, int64_t avail) {
  const float mu = (float)n * (float)sampled / (float)avail;
  return (int)ceilf(mu + 7.0f * sqrtf(mu) + 6.0f);
}

// One thread's share of a stage in flight: 32 fp8 bytes of position t / 4
// (dims (t % 4) * 32 ..) and that position's scale (staged by t % 4 == 0).
struct Ring {
  uint4 r0, r1;
  float s;
};

template <bool kFused>
__global__ void __launch_bounds__(kThreads, 2) logits_kernel(ScanArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t sh_tile[2][kStageBytesBf16];
  __shared__ float sh_scale[2][kStage];
  __shared__ uint32_t sh_hist[kFused ? kWaves : 1][kFused ? kHistBins : 1];
  // a stage's appends, per wave and row, before they go to the global list
  __shared__ float sh_app_score[kFused ? kWaves : 1][kRowsPerWave][kFused ? kAppendCap : 1];
  __shared__ int32_t sh_app_pos[kFused ? kWaves : 1][kRowsPerWave][kFused ? kAppendCap : 1];
  __shared__ int64_t sh_span[2];
  // gate bins per (wave, row) and their (lo, shift); see kGateBins
  __shared__ uint32_t sh_gbins[kFused ? kWaves : 1][kRowsPerWave][kFused ? kGateBins : 1];
  __shared__ uint32_t sh_gpar[kFused ? kWaves : 1][kRowsPerWave][2];
  __shared__ uint32_t sh_redo;   // a calibrated row ended short: the span is scanned again

  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform, so the row indices, ranges and list pointers derived from it live in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t row0 = (int64_t)blockIdx.x * kRowsPerWg;
  const int w = blockIdx.y;

  // The workgroup's span: the union of its rows' ranges, cut to its window.
  if (tid < 64) {
    int64_t lo = INT64_MAX, hi = 0;
    if (tid < kRowsPerWg) {
      const RowRange rr = row_range(a, row0 + tid);
      if (rr.hi > rr.lo) {
        lo = rr.lo;
        hi = rr.hi;
      }
    }
    for (int d = 1; d < kRowsPerWg; d <<= 1) {
      const int64_t l2 = __shfl_xor(lo, d), h2 = __shfl_xor(hi, d);
      lo = l2 < lo ? l2 : lo;
      hi = h2 > hi ? h2 : hi;
    }
    if (tid == 0) {
      const int64_t wlo = (int64_t)w * a.window, whi = wlo + a.window;
      sh_span[0] = lo > wlo ? lo : wlo;
      sh_span[1] = hi < whi ? hi : whi;
      if (kFused) sh_redo = 0;
    }
  }
  __syncthreads();
  // stages start on multiples of 64; windows are multiples of 64 as well, so
  // a stage never reaches into a neighbouring window
  const int64_t span_lo = sh_span[0] & ~(int64_t)(kStage - 1);
  const int64_t span_hi = sh_span[1];

  RowOperand rows[kRowsPerWave];
  RowRange rr[kRowsPerWave];
  int64_t rix[kRowsPerWave];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    rix[i] = row0 + wave * kRowsPerWave + i;
    rr[i] = row_range(a, rix[i]);
    load_row(a.q, a.weights, rix[i], rix[i] < a.num_q, lane, rows[i]);
  }

  // fused scan state, wave-uniform: gate, list length, appends staged in LDS,
  // whether the row's starting gate came from the calibration sample
  uint32_t gate[kRowsPerWave];
  int count[kRowsPerWave];
  int staged[kRowsPerWave];
  bool calibrated[kRowsPerWave];
  if (kFused) {
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      gate[i] = 0;
      count[i] = 0;
      staged[i] = 0;
      calibrated[i] = false;
      if (lane == 0) {
        sh_gpar[wave][i][0] = 0;
        sh_gpar[wave][i][1] = 32;   // no bins before a first trim
      }
    }
  }
  auto list_score = [&](int i) { return a.cand_score + (rix[i] * a.nwin + w) * (int64_t)a.cap; };
  auto list_pos = [&](int i) { return a.cand_pos + (rix[i] * a.nwin + w) * (int64_t)a.cap; };

  if (span_lo < span_hi) {
    const int sn = tid >> 2, sc = tid & 3;
    // The loads are issued unconditionally (a position past the key range
    // reads position num_kv - 1 instead; num_kv >= 1 since the span is not
    // empty): loads under a branch leave the compiler unsure how many are in
    // flight, and its wait for a stage then drains the younger stage too.
    // Scores of such positions are never used: every use checks the row's
    // range, and a stage at or past span_hi is never computed.
    auto fetch = [&](Ring& R, int64_t base) {
      int64_t j = base + sn;
      j = j < a.num_kv ? j : a.num_kv - 1;
      const uint4* src = reinterpret_cast<const uint4*>(a.kv + j * kDim + sc * 32);
      R.r0 = src[0];
      R.r1 = src[1];
      R.s = a.kv_scale[j];
    };
    auto stage = [&](const Ring& R, int buf) {
      uint8_t* t = sh_tile[buf];
      *reinterpret_cast<bf16x8*>(t + tile_offset(sn, 4 * sc)) = widen8(R.r0.x, R.r0.y);
      *reinterpret_cast<bf16x8*>(t + tile_offset(sn, 4 * sc + 1)) = widen8(R.r0.z, R.r0.w);
      *reinterpret_cast<bf16x8*>(t + tile_offset(sn, 4 * sc + 2)) = widen8(R.r1.x, R.r1.y);
      *reinterpret_cast<bf16x8*>(t + tile_offset(sn, 4 * sc + 3)) = widen8(R.r1.z, R.r1.w);
      if (sc == 0) sh_scale[buf][sn] = R.s;
    };
    const int n = lane & 31, hb = lane >> 5;
    auto compute = [&](int64_t base, int buf) {
      bool live = false;
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i) live |= base < rr[i].hi && base + kStage > rr[i].lo;
      if (!live) return;   // wave-uniform
      const uint8_t* t = sh_tile[buf];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int nb = half * kTile + n;
        bf16x8 b[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) b[s] = *reinterpret_cast<const bf16x8*>(t + tile_offset(nb, hb * 8 + s));
        const float scale = sh_scale[buf][nb];
        f32x16 acc[kRowsPerWave];
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) acc[i] = f32x16{};
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
          for (int i = 0; i < kRowsPerWave; ++i)
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rows[i].a[s], b[s], acc[i], 0, 0, 0);
        float score[kRowsPerWave];
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) score[i] = finish_score(rows[i], acc[i], scale, lane);
        const int64_t j = base + nb;
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
          const bool valid = hb == 0 && j >= rr[i].lo && j < rr[i].hi;
          if (!kFused) {
            const int64_t c = j - rr[i].lo;
            if (valid && c < a.logits_stride) a.logits[rix[i] * a.logits_stride + c] = score[i];
          } else {
            // staged in LDS; flush() writes them to the list
            const uint32_t key = order_key(score[i]);
            const bool pass = valid && key >= gate[i];
            const uint64_t m = __ballot(pass);
            if (pass) {
              const int o = staged[i] + wave_prefix(m, lane);
              sh_app_score[wave][i][o] = score[i];
              sh_app_pos[wave][i][o] = (int32_t)j;
            }
            staged[i] += __builtin_popcountll(m);
          }
        }
      }
    };
    // Runs after every stage (at most kStage appends per row).  A row's
    // staged appends go to its list once they could not take another stage,
    // or when the list with them could not (or `all`, at the end); then a
    // list that could not take another stage is trimmed.  Between stages
    // with few appends (after the first fill, a few per stage) nothing is
    // written.  It runs before the next stage's loads are issued: the load
    // counter counts stores too, in issue order, so stores issued after those
    // loads would make the wait for the stage before them wait for them as
    // well.  Either the list is shorter than its window (then it cannot
    // overflow, and a trim happens only above k entries) or its capacity is
    // at least 4k and 4096, so a trim leaves it at most half full.
    auto flush = [&](bool all, int64_t next) {
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i) {
        if (staged[i] == 0) continue;   // wave-uniform
        if (!all && staged[i] <= kAppendCap - kStage && count[i] + staged[i] <= a.cap - kStage) continue;
        for (int e = lane; e < staged[i]; e += 64) {
          list_score(i)[count[i] + e] = sh_app_score[wave][i][e];
          list_pos(i)[count[i] + e] = sh_app_pos[wave][i][e];
        }
        if (__builtin_amdgcn_readfirstlane(sh_gpar[wave][i][1]) < 32)
          gate[i] = raise_gate(sh_app_score[wave][i], staged[i], sh_gbins[wave][i], sh_gpar[wave][i], (uint32_t)a.k,
                               gate[i], lane);
        count[i] += staged[i];
        staged[i] = 0;
        if (count[i] > a.cap - kStage && count[i] > a.k) {
          // gate bins only pay where many positions remain after the trim
          uint32_t* const gb = span_hi - next > 4 * (int64_t)a.cap ? sh_gbins[wave][i] : nullptr;
          const Trimmed t = compact_list(list_score(i), list_pos(i), count[i], (uint32_t)a.k, a.cap / 2, false,
                                         sh_hist[wave], lane, gate[i], gb);
          count[i] = t.count;
          gate[i] = t.gate;
          if (lane == 0) {
            sh_gpar[wave][i][0] = t.bins_lo;
            sh_gpar[wave][i][1] = t.bins_shift;
          }
        }
      }
    };
    // A row's positions in this window, and how many it selects.
    auto row_avail = [&](int i) {
      const int64_t lo = rr[i].lo > span_lo ? rr[i].lo : span_lo;
      const int64_t hi = rr[i].hi < span_hi ? rr[i].hi : span_hi;
      return hi > lo ? hi - lo : (int64_t)0;
    };
    auto row_n = [&](int i) {
      const int64_t av = row_avail(i);
      return av < (int64_t)a.k ? av : (int64_t)a.k;
    };
    // The calibration sample: the middle stage of each of kCalStages equal
    // runs of the span's stages (stage counts fit 32 bits: positions are
    // below 2^31), on spans of at least 4 kCalStages stages whose lists hold
    // the sample without a trim.
    const int nmain = (int)((span_hi - span_lo + kStage - 1) / kStage);
    const bool sampled =
        kFused && nmain >= 4 * kCalStages && a.cap >= kCalStages * kStage + kAppendCap + kStage;
    const int stride = nmain / kCalStages;
    auto sample_base = [&](int idx) { return span_lo + (int64_t)(idx * stride + stride / 2) * kStage; };
    // End of the sample: every sampled position of a row is in its list (the
    // gate was 0, and the capacity holds the sample without a trim).  The
    // row's starting gate is the rank-m sampled key; the list is emptied.
    auto calibrate = [&]() {
      flush(true, span_hi);
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i) {
        const int64_t av = row_avail(i);
        uint32_t g0 = 0;
        bool cal = false;
        if (count[i] > 0 && av > 0) {
          const int m = calibration_rank(row_n(i), count[i], av);
          if (m < count[i]) {
            const Trimmed t = compact_list(list_score(i), list_pos(i), count[i], (uint32_t)m, 0, true, sh_hist[wave],
                                           lane, 0u, nullptr);
            g0 = t.gate > 0u ? t.gate - 1u : 0u;   // the m-th largest sampled key
            cal = true;
          }
        }
        gate[i] = g0;
        count[i] = 0;
        calibrated[i] = cal;
        if (lane == 0) {
          sh_gpar[wave][i][0] = 0;
          sh_gpar[wave][i][1] = 32;
        }
      }
    };
    // After a calibrated pass: a calibrated row with fewer than n entries may
    // have skipped part of its top-n, so every such row is scanned again from
    // gate 0 and the others keep their lists (their ranges are closed for the
    // second pass).  Returns whether a second pass is needed.
    auto verify = [&]() {
      bool failed[kRowsPerWave];
      bool any = false;
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i) {
        failed[i] = calibrated[i] && (int64_t)count[i] < row_n(i);
        any |= failed[i];
      }
      if (any && lane == 0) atomicOr(&sh_redo, 1u);
      __syncthreads();
      const bool redo = __builtin_amdgcn_readfirstlane(sh_redo) != 0u;
      if (redo) {
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
          if (failed[i]) {
            gate[i] = 0;
            count[i] = 0;
            calibrated[i] = false;
            if (lane == 0) {
              sh_gpar[wave][i][0] = 0;
              sh_gpar[wave][i][1] = 32;
            }
          } else {
            rr[i] = RowRange{0, 0};
          }
        }
      }
      return redo;
    };
    if (kFused && sampled) {
      // the sample's stages, pipelined like the scan below (the stages
      // fetched past the sample's end stay in bounds and are never computed)
      Ring r0, r1;
      fetch(r0, sample_base(0));
      stage(r0, 0);
      fetch(r1, sample_base(1));
      fetch(r0, sample_base(2));
      __syncthreads();
      for (int idx = 0; idx < kCalStages; idx += 2) {
        compute(sample_base(idx), 0);
        stage(r1, 1);
        flush(false, span_lo);
        fetch(r1, sample_base(idx + 3));
        __syncthreads();
        compute(sample_base(idx + 1), 1);
        stage(r0, 0);
        flush(false, span_lo);
        fetch(r0, sample_base(idx + 4));
        __syncthreads();
      }
      calibrate();
    }
    // Two stages in flight in registers: the stage computed now, the next one
    // already in LDS, and the two after it loading.  The loop has no exit in
    // its middle (the second stage of a pair past the span is skipped, and
    // its loads stay in bounds): the compiler merges the load counts of every
    // path into the loop head, and an early exit path would make the wait
    // for a stage drain the younger stage as well.  A second pass runs only
    // for rows whose calibrated first pass ended short (verify).
    bool check = kFused && sampled;
    for (;;) {
      Ring r0, r1;
      fetch(r0, span_lo);
      stage(r0, 0);
      fetch(r1, span_lo + kStage);
      fetch(r0, span_lo + 2 * kStage);
      __syncthreads();
      for (int64_t base = span_lo; base < span_hi; base += 2 * kStage) {
        compute(base, 0);
        stage(r1, 1);
        if (kFused) flush(false, base + kStage);
        fetch(r1, base + 3 * kStage);
        __syncthreads();
        if (base + kStage < span_hi) compute(base + kStage, 1);
        stage(r0, 0);
        if (kFused) flush(false, base + 2 * kStage);
        fetch(r0, base + 4 * kStage);
        __syncthreads();
      }
      if (!kFused) break;
      flush(true, span_hi);
      if (!check || !verify()) break;
      check = false;
    }
  }

  if (kFused) {
    // final trim to at most k entries, then hand the list to the row's area;
    // or, with one window per row, only the list's length (the select reads
    // the list where it is)
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      if (rix[i] >= a.num_q) continue;
      if (a.inplace) {
        if (lane == 0) a.row_count[rix[i]] = count[i];
        continue;
      }
      float* lsc = list_score(i);
      int32_t* lps = list_pos(i);
      if (count[i] > a.k)
        count[i] = compact_list(lsc, lps, count[i], (uint32_t)a.k, 0, true, sh_hist[wave], lane, 0u, nullptr).count;
      if (count[i] == 0) continue;
      int off = 0;
      if (lane == 0) off = atomicAdd(&a.row_count[rix[i]], count[i]);
      off = __shfl(off, 0);
      __threadfence();
      float* dsc = a.row_score + rix[i] * a.row_cap + off;
      int32_t* dps = a.row_pos + rix[i] * a.row_cap + off;
      for (int base = 0; base < count[i]; base += 64 * kListBatch) {
        float sv[kListBatch];
        int32_t pv[kListBatch];
#pragma unroll
        for (int b = 0; b < kListBatch; ++b) {
          const int e = base + b * 64 + lane;
          sv[b] = e < count[i] ? lsc[e] : 0.f;
          pv[b] = e < count[i] ? lps[e] : 0;
        }
#pragma unroll
        for (int b = 0; b < kListBatch; ++b) {
          const int e = base + b * 64 + lane;
          if (e < count[i]) {
            dsc[e] = sv[b];
            dps[e] = pv[b];
          }
        }
      }
    }
  }
}

__global__ void zero_counts_kernel(int32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Dense select: each row's clamped range length (the select's seq_len) ...
__global__ void row_lengths_kernel(ScanArgs a, int32_t* len) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r < a.num_q) {
    const RowRange rr = row_range(a, r);
    len[r] = rr.hi > rr.lo ? (int32_t)(rr.hi - rr.lo) : 0;
  }
}

// ... and the select's row-relative positions turned into absolute ones.
__global__ void absolute_positions_kernel(ScanArgs a, const int32_t* rel, int32_t* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < a.num_q * (int64_t)a.k) {
    const int32_t v = rel[i];
    out[i] = v >= 0 ? (int32_t)(row_range(a, i / a.k).lo + v) : -1;
  }
}

hipError_t launch_logits(const ScanArgs& a, int nwin, hipStream_t stream) {
  const dim3 grid((unsigned)((a.num_q + kRowsPerWg - 1) / kRowsPerWg), (unsigned)nwin);
  hipLaunchKernelGGL(logits_kernel<false>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_scan(const ScanArgs& a, int nwin, hipStream_t stream) {
  const int64_t n = a.num_q;
  if (!a.inplace) {   // windows add their counts; in place, every row's count is written
    hipLaunchKernelGGL(zero_counts_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a.row_count, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)((a.num_q + kRowsPerWg - 1) / kRowsPerWg), (unsigned)nwin);
  hipLaunchKernelGGL(logits_kernel<true>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_row_lengths(const ScanArgs& a, int32_t* len, hipStream_t stream) {
  hipLaunchKernelGGL(row_lengths_kernel, dim3((unsigned)((a.num_q + 255) / 256)), dim3(256), 0, stream, a, len);
  return hipGetLastError();
}

hipError_t launch_absolute_positions(const ScanArgs& a, const int32_t* rel, int32_t* out, hipStream_t stream) {
  const int64_t n = a.num_q * (int64_t)a.k;
  hipLaunchKernelGGL(absolute_positions_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a, rel, out);
  return hipGetLastError();
}

int rows_per_workgroup() { return kRowsPerWg; }

}  // namespace indexer
