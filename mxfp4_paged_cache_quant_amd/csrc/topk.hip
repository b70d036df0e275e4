// Per-row top-k over the visible columns [ks, ke) (top_k_per_row of P3
// "SparseAttnIndexerKpool"; exact sets, as P2 "Validation" tests them).
//
// Ranking: value descending, then column ascending; -0.0 == +0.0.  The output
// holds the min(k, n) selected columns followed by -1, in a deterministic
// order: column order, except where the first level's threshold bin is ranked
// directly -- then the keys above that bin come first, in column order, and
// the bin's selected keys follow in rank order -- and for long rows selected
// in one read (the order of the kept pairs, per wave region).
//
// Radix select on order-preserving 32-bit keys with 11-bit digits and one
// workgroup per row (1024 threads for small batches, 512 threads when there
// are many rows).  Each level histograms the next digit of
// the candidate keys in LDS and finds the bin where the running count from
// the top crosses the number still needed; when the digits are exhausted the
// exact k-th key T is known, and a final ordered pass takes every key > T plus
// the lowest-column keys == T.  Output positions come from workgroup prefix
// sums of per-thread counts or from ranks (no atomics), so the output is
// deterministic.  A level costs three barriers: histogram complete, scan
// totals, selection.
//
// The row is held in registers, E keys per thread, with every load of a
// thread issued before any is used (the passes are latency-bound otherwise):
//   * n <= threads*E: one HBM read.  The key range [kmin, kmax] is reduced
//     first and the digits are taken from u = key - kmin, starting at the top
//     bit of kmax - kmin, so the first histogram spreads the row over the bins
//     (fixed top-bit digits would pile similar logits into a few bins).  When
//     the first level's threshold bin holds at most 64 keys (the usual case:
//     2048 bins over the row's own range), those keys are ranked directly and
//     written at their rank, instead of histogramming the remaining digits;
//   * longer rows, in chunks of threads*E: one read when the first chunk
//     predicts the row -- it gives a key with about 1.5 k of the row expected
//     at or above it, one pass keeps every such key in LDS, and the top-k of
//     the kept pairs is the row's when at least k were kept and none
//     overflowed; otherwise two reads: the first histograms the top digit of
//     the keys, the second writes the keys above the threshold bin directly
//     and compacts the bin's (key, column) pairs into LDS (up to 8192, else
//     the remaining levels re-read the row filtered by the bin).
#include <atomic>
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace mxidx {
namespace {

constexpr int kMaxThreads = 1024;
constexpr int kMaxWaves = kMaxThreads / kWave;
constexpr int kCandPairs = 8192;   // (key, column) pairs in dynamic LDS (64 KB), long rows only
constexpr int kWaveHistBins = 2048;

// Threshold bins this small are resolved by ranking their keys pairwise
// (quadratic, so the cutoff is per kernel): the row top-k uses 64, the merge
// of rank lists -- whose first-level bins are larger -- uses 256.
constexpr int kFewCand = 256;      // LDS capacity for the ranked keys
constexpr int kTopkMaxOut = 2048;  // largest k (IDX_TOPK_MAX)
constexpr int kFewTopk = 64;
constexpr int kFewMerge = 256;

template <int BINS>
struct Shared {
  uint32_t hist[BINS];
  uint32_t wave_tot[2][2 * kMaxWaves];  // ping-pong: consecutive scans need one barrier each
  uint32_t sel[3];                      // selected bin, count strictly above it, count in it
  // few-candidate resolve (zeroed at kernel start)
  uint32_t ccount;
  uint32_t ckey[kFewCand], ccol[kFewCand];
};

// Cross-lane steps use DPP row shifts (lane i reads lane i - d of its 16-lane
// row; a source outside the row reads as 0) and lane reads into scalars, not
// LDS permutes: each step is a few VALU cycles instead of an LDS round trip.
// Callers run them with every lane of the wave active.
__device__ __forceinline__ uint32_t row_shr(uint32_t x, int d) {
  switch (d) {
    case 1: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);
    case 2: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);
    case 4: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);
    default: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);
  }
}

// Sum over each aligned group of SPAN lanes (SPAN a power of two <= 16),
// complete in the group's last lane.
template <int SPAN>
__device__ __forceinline__ uint32_t group_sum(uint32_t x) {
  static_assert(SPAN >= 1 && SPAN <= 16 && (SPAN & (SPAN - 1)) == 0, "groups within a DPP row");
#pragma unroll
  for (int d = 1; d < SPAN; d <<= 1) x += row_shr(x, d);
  return x;
}

// Inclusive prefix sum over the wave in lane order.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x = group_sum<16>(x);                          // inclusive within each row
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
  const int lane = threadIdx.x & 63;
  return x + (lane >= 16 ? r0 : 0u) + (lane >= 32 ? r1 : 0u) + (lane >= 48 ? r2 : 0u);
}

// Maximum over the wave (uniform result).
__device__ __forceinline__ uint32_t wave_umax(uint32_t x) {
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) x = max(x, row_shr(x, d));   // 0 from outside a row is neutral
  const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)x, 15),
                         (uint32_t)__builtin_amdgcn_readlane((int)x, 31));
  const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)x, 47),
                         (uint32_t)__builtin_amdgcn_readlane((int)x, 63));
  return max(a, b);
}

// Exclusive prefix sum over the workgroup in thread order; also returns the
// total.  One barrier; consecutive calls must alternate `parity`.
template <int NT, int BINS>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, Shared<BINS>& s, int parity,
                                               uint32_t& total) {
  constexpr int kWaves = NT / kWave;
  static_assert(kWaves <= 16, "the wave totals are scanned in one DPP row");
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t x = wave_incl_scan(v);
  uint32_t* wt = s.wave_tot[parity];
  if (lane == 63) wt[wid] = x;
  __syncthreads();
  // lane i < kWaves takes wave i's total; their running sums give each wave its base
  const uint32_t w = group_sum<16>(lane < kWaves ? wt[lane & 15] : 0u);
  const uint32_t before = wid ? (uint32_t)__builtin_amdgcn_readlane((int)w, wid - 1) : 0u;
  total = (uint32_t)__builtin_amdgcn_readlane((int)w, kWaves - 1);
  return before + x - v;
}

// Bin b (from the top) with count(bins > b) < need <= count(bins >= b); needs
// need >= 1 and a histogram total >= need.  Sets s.sel = {b, count above b}
// and leaves the histogram cleared for the next level.  Two barriers.
template <int NT, int BINS>
__device__ void select_bin(Shared<BINS>& s, uint32_t need, int parity) {
  constexpr int per = BINS / NT;                 // bins per thread, descending
  const int top = BINS - 1 - per * (int)threadIdx.x;
  uint32_t c[per];
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < per; ++j) {
    c[j] = s.hist[top - j];
    sum += c[j];
  }
  uint32_t total;
  uint32_t run = block_scan<NT>(sum, s, parity, total);
#pragma unroll
  for (int j = 0; j < per; ++j) {
    if (run < need && run + c[j] >= need) {
      s.sel[0] = (uint32_t)(top - j);
      s.sel[1] = run;
      s.sel[2] = c[j];
    }
    run += c[j];
    s.hist[top - j] = 0;                          // every read of the histogram is done
  }
  __syncthreads();
}

// select_bin with one barrier: after the wave totals are published, every
// wave finds the wave whose share of the bins holds the crossing and scans
// that share itself (two bins per lane at 1024 threads), so the selected bin,
// the count above it and its own count reach every wave in scalar registers
// without a second barrier.  The histogram is left as it is (a caller that
// histograms again must clear it behind a barrier).  Same preconditions.
template <int NT, int BINS>
__device__ __forceinline__ void select_bin_wave(Shared<BINS>& s, uint32_t need, int parity,
                                                uint32_t& bin, uint32_t& above, uint32_t& inbin) {
  constexpr int per = BINS / NT;
  constexpr int kWaves = NT / kWave;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int top = BINS - 1 - per * (int)threadIdx.x;
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < per; ++j) sum += s.hist[top - j];
  const uint32_t x = wave_incl_scan(sum);
  uint32_t* wt = s.wave_tot[parity];
  if (lane == 63) wt[wid] = x;
  __syncthreads();
  // running totals over the waves (lane i: waves 0..i), then the first wave
  // whose running total reaches `need`
  const uint32_t w = group_sum<16>(lane < kWaves ? wt[lane & 15] : 0u);
  const uint64_t hit = __ballot(lane < kWaves && w >= need);
  const int ws = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
  const uint32_t base = ws ? (uint32_t)__builtin_amdgcn_readlane((int)w, ws - 1) : 0u;
  const int top2 = BINS - 1 - per * (ws * kWave + lane);
  uint32_t c[per];
  uint32_t sum2 = 0;
#pragma unroll
  for (int j = 0; j < per; ++j) {
    c[j] = s.hist[top2 - j];
    sum2 += c[j];
  }
  uint32_t run = base + wave_incl_scan(sum2) - sum2;
  const uint64_t hl = __ballot(run < need && run + sum2 >= need);
  const int ls = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hl));
  uint32_t b = 0, r = 0, n = 0;
#pragma unroll
  for (int j = 0; j < per; ++j) {
    if (run < need && run + c[j] >= need) {
      b = (uint32_t)(top2 - j);
      r = run;
      n = c[j];
    }
    run += c[j];
  }
  bin = (uint32_t)__builtin_amdgcn_readlane((int)b, ls);
  above = (uint32_t)__builtin_amdgcn_readlane((int)r, ls);
  inbin = (uint32_t)__builtin_amdgcn_readlane((int)n, ls);
}

template <int NT, int BINS>
__device__ __forceinline__ void clear_hist(Shared<BINS>& s) {
  for (int i = threadIdx.x; i < BINS; i += NT) s.hist[i] = 0;
}

// Per-slot loops run as f(std::true_type) on a wave whose E*64 slots all hold
// keys of the row -- the per-slot validity tests then fold away (on a 8192-key
// row they cost about a tenth of the kernel) -- and as f(std::false_type) on
// the wave that holds the row's end or lies past it.  `wave_full` is uniform
// over the wave, so each wave runs one of the two bodies.
template <typename F>
__device__ __forceinline__ void per_fill(bool wave_full, F&& f) {
  if (wave_full) f(std::true_type{});
  else f(std::false_type{});
}

// Keys E*t + e (e < E) of the segment src[0, n) into thread t's registers;
// returns how many are valid.  All loads are issued before any is used.
template <int E>
__device__ __forceinline__ int load_keys(const float* __restrict__ src, int64_t n, bool vec,
                                         uint32_t (&key)[E]) {
  const int64_t first = (int64_t)E * threadIdx.x;
  const int nv = (int)max((int64_t)0, min((int64_t)E, n - first));
  if (vec && nv == E) {
    uint4 v[E / 4];
#pragma unroll
    for (int q = 0; q < E / 4; ++q) v[q] = *reinterpret_cast<const uint4*>(src + first + 4 * q);
#pragma unroll
    for (int q = 0; q < E / 4; ++q) {
      key[4 * q + 0] = f32_key(v[q].x);
      key[4 * q + 1] = f32_key(v[q].y);
      key[4 * q + 2] = f32_key(v[q].z);
      key[4 * q + 3] = f32_key(v[q].w);
    }
  } else {
    uint32_t raw[E];
#pragma unroll
    for (int e = 0; e < E; ++e) raw[e] = (e < nv) ? __float_as_uint(src[first + e]) : 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) key[e] = f32_key(raw[e]);
  }
  return nv;
}

// Keys c0 + E*t + e of a chunk that lies wholly inside a 16-byte aligned row:
// E/4 vector loads, no branch.
template <int E>
__device__ __forceinline__ void load_full(const float* __restrict__ src, int64_t c0,
                                          uint32_t (&key)[E]) {
  const float* p = src + c0 + (int64_t)E * threadIdx.x;
  uint4 v[E / 4];
#pragma unroll
  for (int q = 0; q < E / 4; ++q) v[q] = *reinterpret_cast<const uint4*>(p + 4 * q);
#pragma unroll
  for (int q = 0; q < E / 4; ++q) {
    key[4 * q + 0] = f32_key(v[q].x);
    key[4 * q + 1] = f32_key(v[q].y);
    key[4 * q + 2] = f32_key(v[q].z);
    key[4 * q + 3] = f32_key(v[q].w);
  }
}

// Runs body(c0, key, nv) over the chunks of C = NT*E keys of src[0, n) in
// order.  The full chunks of an aligned row are double-buffered: the next
// chunk's loads are issued before a chunk is processed (the refill is
// unconditional -- past the last full chunk it re-reads that chunk -- so the
// waits on it are exact); a partial last chunk, and every chunk of an
// unaligned row, use the generic loader.
template <int NT, int E, typename Body>
__device__ __forceinline__ void for_chunks(const float* __restrict__ src, int64_t n, bool vec,
                                           Body&& body) {
  constexpr int64_t C = (int64_t)NT * E;
  const int64_t nfull = vec ? n / C : 0;
  if (nfull > 0) {
    uint32_t ka[E], kb[E];
    load_full<E>(src, 0, ka);
    int64_t i = 0;
    for (; i + 1 < nfull; i += 2) {
      load_full<E>(src, (i + 1) * C, kb);
      body(i * C, ka, E);
      load_full<E>(src, min(i + 2, nfull - 1) * C, ka);
      body((i + 1) * C, kb, E);
    }
    if (i < nfull) body(i * C, ka, E);
  }
  for (int64_t c0 = nfull * C; c0 < n; c0 += C) {
    uint32_t key[E];
    const int nv = load_keys<E>(src + c0, n - c0, vec, key);
    body(c0, key, nv);
  }
}

// One radix level over register-held keys: u = key - kmin; candidates have
// u >> shift == prefix (all when shift >= 32); digit = bits shift-1 .. nsh.
template <int E, int BINS>
__device__ __forceinline__ void hist_level(Shared<BINS>& s, const uint32_t (&key)[E], int nv,
                                           uint32_t kmin, int shift, uint32_t prefix, int nsh,
                                           uint32_t dmask, bool wfull = false) {
  per_fill(wfull, [&](auto full) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t u = key[e] - kmin;
      if ((full.value || e < nv) && (shift >= 32 || (u >> shift) == prefix))
        atomicAdd(&s.hist[(u >> nsh) & dmask], 1u);
    }
  });
}

// First level over the key range: u = key - kmin < 2^(nsh + digit bits), so
// every valid key counts and its digit is u >> nsh.
template <int E, int BINS>
__device__ __forceinline__ void hist_first(Shared<BINS>& s, const uint32_t (&key)[E], int nv,
                                           uint32_t kmin, int nsh, bool wfull = false) {
  per_fill(wfull, [&](auto full) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (full.value || e < nv) atomicAdd(&s.hist[(key[e] - kmin) >> nsh], 1u);
  });
}

template <int BINS>
constexpr int digit_bits() {
  int b = 0;
  while ((1 << b) < BINS) ++b;
  return b;
}

// Levels from `shift` down to bit 0 on register-held keys (histogram clear on
// entry).  Returns u_t (the exact threshold, as key - kmin) and how many keys
// equal to it to take.
template <int NT, int BINS, int E>
__device__ __forceinline__ void refine_regs(Shared<BINS>& s, const uint32_t (&key)[E], int nv,
                                            uint32_t kmin, int shift, uint32_t prefix,
                                            uint32_t need, int& parity, uint32_t& u_t,
                                            uint32_t& need_ties, bool wfull = false) {
  constexpr int D = digit_bits<BINS>();
  while (shift > 0) {
    const int nsh = shift > D ? shift - D : 0;
    const uint32_t dmask = (1u << (shift - nsh)) - 1u;
    hist_level(s, key, nv, kmin, shift, prefix, nsh, dmask, wfull);
    __syncthreads();
    select_bin<NT>(s, need, parity);
    parity ^= 1;
    need -= s.sel[1];
    prefix = (prefix << (shift - nsh)) | s.sel[0];
    shift = nsh;
  }
  u_t = prefix;
  need_ties = need;
}

// Output of the row when the threshold bin (keys with u >> shift == prefix)
// holds at most FEW keys and the `need`-th largest of them is the k-th of the
// row.  Keys in higher bins (`above` of them) go to out[0, above) in thread
// order, from one prefix sum whose barrier also publishes the bin's gathered
// (key, column) pairs; each bin key is then ranked directly -- rank = number
// of bin keys before it in (key desc, column asc) order, counted pairwise by
// kPerCand threads and summed over their DPP row -- and written to
// out[above + rank] when rank < need.  Two barriers, no remaining digits and
// no further pass.  Columns are col0 + e, or cols[e] when kCols.
template <int NT, int FEW, bool kCols, int BINS, int E>
__device__ __forceinline__ void select_few(Shared<BINS>& s, const uint32_t (&key)[E],
                                           const uint32_t (&cols)[E], int nv, uint32_t col0,
                                           uint32_t kmin, int shift, uint32_t prefix,
                                           uint32_t need, uint32_t above,
                                           int32_t* __restrict__ out, int parity,
                                           bool wfull = false) {
  static_assert(FEW <= kFewCand && NT % FEW == 0, "ranked keys: LDS capacity, threads");
  constexpr int kPerCand = NT / FEW;             // threads per candidate
  constexpr int kJ = FEW / kPerCand;             // comparisons per thread
  uint32_t ca = 0;
  per_fill(wfull, [&](auto full) __attribute__((always_inline)) {
    uint32_t a = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t d = (key[e] - kmin) >> shift;
      const bool ok = full.value || e < nv;
      if (ok && d > prefix) ++a;
      if (ok && d == prefix) {
        const uint32_t slot = atomicAdd(&s.ccount, 1u);
        s.ckey[slot] = key[e];
        s.ccol[slot] = kCols ? cols[e] : col0 + (uint32_t)e;
      }
    }
    ca = a;
  });
  uint32_t total;
  const uint32_t pos = block_scan<NT>(ca, s, parity, total);
  // With 16 or more keys per thread the row's k outputs are staged in the
  // histogram's words (no wave reads the histogram past the scan's barrier)
  // and stored in one coalesced pass: the per-thread positions scatter over
  // the row, a global store per key slot against an LDS write (prefill-chunk
  // rows 76.0 -> 57.4 us).  With 8 keys per thread (decode rows) the stores go
  // out directly: the staging's extra barrier costs more (5.57 -> 5.63 us).
  constexpr bool kStage = E >= 16;
  static_assert(!kStage || BINS >= kTopkMaxOut, "the staging area holds a whole output row");
  uint32_t* stage = s.hist;
  auto emit = [&](uint32_t o, uint32_t c) __attribute__((always_inline)) {
    if constexpr (kStage) stage[o] = c;
    else out[o] = (int32_t)c;
  };
  per_fill(wfull, [&](auto full) __attribute__((always_inline)) {
    uint32_t p = pos;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if ((full.value || e < nv) && ((key[e] - kmin) >> shift) > prefix)
        emit(p++, kCols ? cols[e] : col0 + (uint32_t)e);
  });
  const uint32_t cnt = s.ccount;
  const uint32_t i = threadIdx.x / kPerCand;
  const uint32_t j0 = (threadIdx.x % kPerCand) * kJ;
  uint32_t ki = 0, ci = 0, before = 0;
  if (i < cnt) {
    ki = s.ckey[i];
    ci = s.ccol[i];
    if constexpr (kJ <= 8) {
      // a few comparisons per thread: unrolled, their LDS reads in flight together
#pragma unroll
      for (int jj = 0; jj < kJ; ++jj) {
        const uint32_t j = j0 + jj;
        if (j < cnt) {
          const uint32_t kj = s.ckey[j], cj = s.ccol[j];
          before += (kj > ki || (kj == ki && cj < ci)) ? 1u : 0u;
        }
      }
    } else {
      // a long share (the 256-key ranking): bounded by the bin's size, which is
      // usually a few keys, instead of testing every slot of the share
      const uint32_t jn = cnt > j0 ? min((uint32_t)kJ, cnt - j0) : 0u;
      for (uint32_t jj = 0; jj < jn; ++jj) {
        const uint32_t kj = s.ckey[j0 + jj], cj = s.ccol[j0 + jj];
        before += (kj > ki || (kj == ki && cj < ci)) ? 1u : 0u;
      }
    }
  }
  before = group_sum<kPerCand>(before);          // a candidate's threads share a DPP row
  if (i < cnt && threadIdx.x % kPerCand == kPerCand - 1 && before < need) emit(above + before, ci);
  if constexpr (kStage) {
    __syncthreads();
    // above + need outputs: the keys above the bin and the bin's first `need`
    for (uint32_t o = threadIdx.x; o < above + need; o += NT) out[o] = (int32_t)stage[o];
  }
}

// Ordered output of register-held candidates (thread t holds consecutive
// candidates, so thread order is candidate order): every u > u_t, and the
// first need_ties with u == u_t, at out[base + rank].  Candidates are the
// valid keys (with key >> fshift == fbin when filt).  gt_run / tie_run carry
// the counts of earlier chunks and are advanced by this chunk's totals.
template <int NT, bool kCols, int BINS, int E>
__device__ __forceinline__ void emit_regs(Shared<BINS>& s, const uint32_t (&key)[E],
                                          const uint32_t (&cols)[E], int64_t col0, int nv,
                                          uint32_t kmin, uint32_t u_t, uint32_t need_ties,
                                          bool filt, int fshift, uint32_t fbin,
                                          int32_t* __restrict__ out, uint32_t base, int k,
                                          int& parity, uint32_t& gt_run, uint32_t& tie_run,
                                          bool wfull = false) {
  uint32_t cg = 0, ct = 0;
  per_fill(wfull, [&](auto full) __attribute__((always_inline)) {
    uint32_t a = 0, b = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t u = key[e] - kmin;
      const bool ok = (full.value || e < nv) && (!filt || (key[e] >> fshift) == fbin);
      a += (ok && u > u_t) ? 1u : 0u;
      b += (ok && u == u_t) ? 1u : 0u;
    }
    cg = a;
    ct = b;
  });
  uint32_t total;
  const uint32_t pre = block_scan<NT>(cg | (ct << 16), s, parity, total);
  parity ^= 1;
  const uint32_t g = gt_run + (pre & 0xffffu);
  const uint32_t t = tie_run + (pre >> 16);
  // (the lambdas below update copies: a captured counter incremented on two
  // paths would be addressed through a pointer select and live in scratch)
  per_fill(wfull, [&](auto full) __attribute__((always_inline)) {
    uint32_t gl = g, tl = t;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t u = key[e] - kmin;
      const bool ok = (full.value || e < nv) && (!filt || (key[e] >> fshift) == fbin);
      const int64_t col = kCols ? (int64_t)cols[e] : col0 + e;
      if (ok && u > u_t) {
        const uint32_t pos = base + gl + min(tl, need_ties);
        if (pos < (uint32_t)k) out[pos] = (int32_t)col;
        ++gl;
      } else if (ok && u == u_t) {
        if (tl < need_ties && base + gl + tl < (uint32_t)k) out[base + gl + tl] = (int32_t)col;
        ++tl;
      }
    }
  });
  gt_run += total & 0xffffu;
  tie_run += total >> 16;
}

// Top-k of register-held (key, column) pairs: slots e < nv of each thread, of
// which those with okmask bit e set are valid (the others take part as
// (kmin, 0xffffffff), below every valid pair).  Ranking: key descending, then
// column ascending.  Writes the min(k, valid) selected columns to out[0, k),
// then -1; the order is deterministic.  Starts with the histogram cleared,
// ccount zero, and a barrier after the caller's last scan.
template <int NT, int FEW, int BINS, int E>
__device__ __forceinline__ void select_pairs_ranged(Shared<BINS>& s, uint32_t (&key)[E],
                                                    const uint32_t (&col)[E], uint32_t okmask,
                                                    int nv, int k, int32_t* __restrict__ out,
                                                    int parity, uint32_t kmin, uint32_t kmax,
                                                    uint32_t total_valid);

template <int NT, int FEW, int BINS, int E>
__device__ __forceinline__ void select_pairs(Shared<BINS>& s, uint32_t (&key)[E],
                                             const uint32_t (&col)[E], uint32_t okmask, int nv,
                                             int k, int32_t* __restrict__ out, int parity) {
  constexpr int kWaves = NT / kWave;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  // valid count and key range over the valid candidates
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if ((okmask >> e) & 1u) {
      kmin = min(kmin, key[e]);
      kmax = max(kmax, key[e]);
    }
  kmin = ~wave_umax(~kmin);
  kmax = wave_umax(kmax);
  // the wave ranges go to the buffer the scan below does not write (the
  // caller's last scan, if any, used it and has passed a barrier since)
  uint32_t* wr = s.wave_tot[parity ^ 1];
  if (lane == 0) {
    wr[wid] = kmin;
    wr[kMaxWaves + wid] = kmax;
  }
  uint32_t total_valid;
  (void)block_scan<NT>((uint32_t)__popc(okmask), s, parity, total_valid);   // one barrier
  parity ^= 1;
  kmin = ~wave_umax(lane < kWaves ? ~wr[lane & 15] : 0u);
  kmax = wave_umax(lane < kWaves ? wr[kMaxWaves + (lane & 15)] : 0u);
  __syncthreads();                              // the next scan rewrites that buffer
  select_pairs_ranged<NT, FEW>(s, key, col, okmask, nv, k, out, parity, kmin, kmax, total_valid);
}

// select_pairs once the valid count and bounds of the valid keys are known:
// kmin <= every valid key <= kmax (bounds, not necessarily attained).  Starts
// like select_pairs, after a barrier that follows the caller's last scan.
template <int NT, int FEW, int BINS, int E>
__device__ __forceinline__ void select_pairs_ranged(Shared<BINS>& s, uint32_t (&key)[E],
                                                    const uint32_t (&col)[E], uint32_t okmask,
                                                    int nv, int k, int32_t* __restrict__ out,
                                                    int parity, uint32_t kmin, uint32_t kmax,
                                                    uint32_t total_valid) {
  if (total_valid <= (uint32_t)k) {             // every valid candidate, then -1
    uint32_t tot;
    uint32_t pos = block_scan<NT>((uint32_t)__popc(okmask), s, parity, tot);
#pragma unroll
    for (int e = 0; e < E; ++e)
      if ((okmask >> e) & 1u) out[pos++] = (int32_t)col[e];
    for (uint32_t i = tot + threadIdx.x; i < (uint32_t)k; i += NT) out[i] = -1;
    return;
  }
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (!((okmask >> e) & 1u)) key[e] = kmin;   // empty: (kmin, 0xffffffff), below every valid one

  uint32_t key_t, col_t;
  bool col_known = false;
  uint32_t u_t = 0, need_ties = (uint32_t)k;
  const uint32_t range = kmax - kmin;
  const int L = range ? 32 - __clz(range) : 0;
  if (L > 0) {
    constexpr int D = digit_bits<BINS>();
    const int nsh = L > D ? L - D : 0;
    hist_first(s, key, nv, kmin, nsh);
    __syncthreads();
    select_bin<NT>(s, (uint32_t)k, parity);
    parity ^= 1;
    const uint32_t need = (uint32_t)k - s.sel[1];
    const uint32_t bin = s.sel[0];
    if (nsh == 0) {
      u_t = bin;
      need_ties = need;
    } else if (s.sel[2] <= (uint32_t)FEW) {
      select_few<NT, FEW, true>(s, key, col, nv, 0u, kmin, nsh, bin, need,
                                      (uint32_t)k - need, out, parity);
      return;
    } else {
      refine_regs<NT>(s, key, nv, kmin, nsh, bin, need, parity, u_t, need_ties);
    }
    // the last radix level's bin holds exactly the keys equal to the threshold:
    // when all of them are taken, no column select is needed
    if (!col_known && s.sel[2] == need_ties) {
      col_t = 0xfffffffeu;                      // every valid column (empty slots are 0xffffffff)
      col_known = true;
    }
  }
  key_t = kmin + u_t;
  if (!col_known) {
    // the need_ties lowest columns among the keys equal to key_t: largest ~column
    uint32_t key2[E];
#pragma unroll
    for (int e = 0; e < E; ++e) key2[e] = (e < nv && key[e] == key_t) ? ~col[e] : 0u;
    uint32_t u2, n2;
    refine_regs<NT>(s, key2, nv, 0u, 32, 0u, need_ties, parity, u2, n2);
    col_t = ~u2;
  }
  // ordered output of every candidate at or above (key_t, col_t)
  uint32_t cnt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e)
    cnt += (e < nv && (key[e] > key_t || (key[e] == key_t && col[e] <= col_t))) ? 1u : 0u;
  uint32_t tot;
  uint32_t pos = block_scan<NT>(cnt, s, parity, tot);
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (e < nv && (key[e] > key_t || (key[e] == key_t && col[e] <= col_t))) {
      if (pos < (uint32_t)k) out[pos] = (int32_t)col[e];
      ++pos;
    }
}

// Top-k of row r by one workgroup.  kLong = false: only rows that fit in
// registers (the long-row code, and its registers, are left out); kLong =
// true needs `dyn` = 64 KB of LDS.
template <int NT, int E, int BINS, bool kLong>
__device__ __forceinline__ void topk_row(Shared<BINS>& s, uint32_t* __restrict__ dyn,
                                         const float* __restrict__ logits, int64_t ld, int64_t r,
                                         const int32_t* __restrict__ ks,
                                         const int32_t* __restrict__ ke, int k,
                                         int32_t* __restrict__ out_idx) {
  constexpr int kWaves = NT / kWave;
  constexpr int64_t C = (int64_t)NT * E;          // keys held per pass
  const float* row = logits + r * ld;
  int32_t* out = out_idx + r * (int64_t)k;
  const int64_t lo = ks ? max((int64_t)ks[r], (int64_t)0) : 0;
  const int64_t hi = min((int64_t)ke[r], ld);
  const int64_t n = hi > lo ? hi - lo : 0;

  if (n <= k) {
    for (int i = threadIdx.x; i < k; i += NT) out[i] = (i < n) ? (int32_t)(lo + i) : -1;
    return;
  }
  const float* src = row + lo;
  const bool vec = (reinterpret_cast<uintptr_t>(src) & 15) == 0;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  int parity = 0;
  if (threadIdx.x == 0) s.ccount = 0;           // read only after later barriers

  if (n <= C) {
    // ---- the whole row in registers: one read ----
    // A row of exactly C keys runs with every wave full at compile time.
    auto row_regs = [&](auto all_full) __attribute__((always_inline)) {
      uint32_t key[E];
      const int wfirst = __builtin_amdgcn_readfirstlane(threadIdx.x) & ~(kWave - 1);
      // every slot of the wave valid (a constant on a row of exactly C keys)
      const bool wfull = all_full.value || n >= (int64_t)(wfirst + kWave) * E;
      int nv = E;
      if (wfull && vec) load_full<E>(src, 0, key);
      else nv = load_keys<E>(src, n, vec, key);
      clear_hist<NT>(s);                            // overlaps the loads
      uint32_t kmin = 0xffffffffu, kmax = 0u;
      per_fill(wfull, [&](auto full) __attribute__((always_inline)) {
        uint32_t lo_k = 0xffffffffu, hi_k = 0u;
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (full.value || e < nv) {
            lo_k = min(lo_k, key[e]);
            hi_k = max(hi_k, key[e]);
          }
        kmin = lo_k;
        kmax = hi_k;
      });
      kmin = ~wave_umax(~kmin);
      kmax = wave_umax(kmax);
      if (lane == 0) {
        s.wave_tot[1][wid] = kmin;
        s.wave_tot[1][kMaxWaves + wid] = kmax;
      }
      __syncthreads();
      kmin = ~wave_umax(lane < kWaves ? ~s.wave_tot[1][lane & 15] : 0u);
      kmax = wave_umax(lane < kWaves ? s.wave_tot[1][kMaxWaves + (lane & 15)] : 0u);
      // wave_tot[1] is next written by the second scan, after at least one more barrier
      const uint32_t range = kmax - kmin;
      const int L = range ? 32 - __clz(range) : 0;     // bit length of the key range
      uint32_t u_t = 0, need_ties = (uint32_t)k;        // all keys equal: the lowest columns
      if (L > 0) {
        // first digit over the whole range, then either a direct ranking of a
        // small threshold bin or the remaining digits
        constexpr int D = digit_bits<BINS>();
        const int nsh = L > D ? L - D : 0;
        hist_first(s, key, nv, kmin, nsh, wfull);
        __syncthreads();
        uint32_t bin, above, inbin;
        select_bin_wave<NT>(s, (uint32_t)k, parity, bin, above, inbin);
        parity ^= 1;
        const uint32_t need = (uint32_t)k - above;
        if (nsh == 0) {
          u_t = bin;
          need_ties = need;
        } else if (inbin <= (uint32_t)kFewTopk) {
          select_few<NT, kFewTopk, false>(s, key, key, nv, (uint32_t)(lo + (int64_t)E * threadIdx.x),
                                          kmin, nsh, bin, need, above, out, parity, wfull);
          return;
        } else {
          // every wave has read its share of the histogram: clear it for the
          // remaining digits
          __syncthreads();
          clear_hist<NT>(s);
          __syncthreads();
          refine_regs<NT>(s, key, nv, kmin, nsh, bin, need, parity, u_t, need_ties, wfull);
        }
      }
      uint32_t gr = 0, tr = 0;
      emit_regs<NT, false>(s, key, key, lo + (int64_t)E * threadIdx.x, nv, kmin, u_t, need_ties,
                           false, 0, 0u, out, 0u, k, parity, gr, tr, wfull);
    };
    // (only in the 1024-thread kernels, launched for few rows: the third copy
    // of the per-slot loops costs registers, which the many-row kernels spend
    // on occupancy)
    if constexpr (NT == kMaxThreads) {
      if (n == C) {
        row_regs(std::true_type{});
        return;
      }
    }
    row_regs(std::false_type{});
    return;
  }
  if constexpr (kLong) {
    // ---- long row, chunks of C keys ----
    // One read when an estimate holds: the first chunk gives a key t_est with
    // about 1.5 k of the row's keys expected at or above it (one histogram level
    // over the chunk's own range); one pass then keeps every key >= t_est, each
    // wave appending to its own region of the pair buffer in row order (a ballot
    // prefix, no atomics, no barriers).  With at least k keys kept and no region
    // full, the row's top-k is the top-k of the kept pairs.  Otherwise (a row
    // whose first chunk misrepresents it) the two-pass path below runs.
    {
      constexpr int kRegion = kCandPairs / kWaves;  // pairs per wave
      constexpr int E2 = kRegion / kWave;           // kept pairs per thread afterwards
      uint32_t* ck = dyn;
      uint32_t* cc = dyn + kCandPairs;
      // t_est from a full first chunk: about 1.5 k of the row's keys are
      // expected at or above it
      auto estimate = [&](const uint32_t (&key)[E]) __attribute__((always_inline)) -> uint32_t {
        clear_hist<NT>(s);
        uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          kmin = min(kmin, key[e]);
          kmax = max(kmax, key[e]);
        }
        kmin = ~wave_umax(~kmin);
        kmax = wave_umax(kmax);
        if (lane == 0) {
          s.wave_tot[1][wid] = kmin;
          s.wave_tot[1][kMaxWaves + wid] = kmax;
        }
        __syncthreads();
        kmin = ~wave_umax(lane < kWaves ? ~s.wave_tot[1][lane & 15] : 0u);
        kmax = wave_umax(lane < kWaves ? s.wave_tot[1][kMaxWaves + (lane & 15)] : 0u);
        const uint32_t range = kmax - kmin;
        const int L = range ? 32 - __clz(range) : 0;
        constexpr int D = digit_bits<BINS>();
        const int nsh = L > D ? L - D : 0;
        hist_first(s, key, E, kmin, nsh);
        __syncthreads();
        const int64_t want = ((int64_t)3 * k * C) / (2 * n) + 32;   // of the chunk's C keys
        select_bin<NT>(s, (uint32_t)min(want, C), parity);
        parity ^= 1;
        return kmin + (s.sel[0] << nsh);            // lower edge of that key's bin
      };
      uint32_t t_est;
      uint32_t kept = 0;                            // this wave's pairs (wave-uniform)
      uint32_t* wk = ck + wid * kRegion;
      uint32_t* wc = cc + wid * kRegion;
      // one pass keeps every key >= t_est, each wave appending to its region
      auto keep = [&](int64_t c0, const uint32_t (&key)[E], int nv) __attribute__((always_inline)) {
        const uint32_t col0 = (uint32_t)(lo + c0 + (int64_t)E * threadIdx.x);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const bool take = e < nv && key[e] >= t_est;
          const uint64_t m = __ballot(take);
          if (m) {                                  // wave-uniform
            const uint32_t pos = kept + __builtin_amdgcn_mbcnt_hi(
                                            (uint32_t)(m >> 32),
                                            __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (take && pos < (uint32_t)kRegion) {
              wk[pos] = key[e];
              wc[pos] = col0 + (uint32_t)e;
            }
            kept += (uint32_t)__popcll(m);
          }
        }
      };
      if (vec) {
        // Aligned row: the estimate's chunk 0 stays in registers for the pass
        // (it is not read twice) and chunk 1 loads during the estimate; then
        // two buffers, each refilled right after use (refills past the last
        // full chunk re-read it, so waits stay exact).  A third buffer was
        // measured: it slowed the estimate's own chunk more than it sped the
        // pass, whose ballot bookkeeping, not memory, sets its pace.
        const int64_t nfull = n / C;                // >= 1
        uint32_t ka[E], kb[E];
        load_full<E>(src, 0, ka);
        load_full<E>(src, min((int64_t)1, nfull - 1) * C, kb);
        t_est = estimate(ka);
        int64_t i = 0;
        for (; i + 1 < nfull; i += 2) {
          keep(i * C, ka, E);
          load_full<E>(src, min(i + 2, nfull - 1) * C, ka);
          keep((i + 1) * C, kb, E);
          load_full<E>(src, min(i + 3, nfull - 1) * C, kb);
        }
        if (i < nfull) keep(i * C, ka, E);
        for (int64_t c0 = nfull * C; c0 < n; c0 += C) {
          uint32_t key[E];
          const int nv = load_keys<E>(src + c0, n - c0, vec, key);
          keep(c0, key, nv);
        }
      } else {
        {
          uint32_t key[E];
          (void)load_keys<E>(src, n, vec, key);     // n > C: a full chunk
          t_est = estimate(key);
        }
        for_chunks<NT, E>(src, n, vec, keep);
      }
      if (lane == 0) s.wave_tot[0][wid] = kept;
      __syncthreads();
      uint32_t total = 0, fullest = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        total += s.wave_tot[0][w];
        fullest = max(fullest, s.wave_tot[0][w]);
      }
      if (total >= (uint32_t)k && fullest <= (uint32_t)kRegion) {
        // a wave's kept pairs are a prefix of its region, so each lane's valid
        // slots are a prefix of its E2: passing their count (not E2) keeps the
        // empty slots out of every histogram (as the range minimum they would
        // all hit one bin, and those LDS atomics serialize)
        uint32_t key[E2], col[E2];
        uint32_t okmask = 0;
        const int nv2 = (int)min((uint32_t)E2, kept - min(kept, (uint32_t)(lane * E2)));
#pragma unroll
        for (int e = 0; e < E2; ++e) {
          const uint32_t i = (uint32_t)(lane * E2 + e);
          key[e] = e < nv2 ? wk[i] : 0u;
          col[e] = e < nv2 ? wc[i] : 0xffffffffu;
          okmask |= (e < nv2 ? 1u : 0u) << e;
        }
        __syncthreads();                            // every count read before the next scans
        select_pairs<NT, kFewMerge>(s, key, col, okmask, nv2, k, out, parity);
        return;
      }
      __syncthreads();                              // counts read before the buffers are reused
    }
    // Pass 1: histogram of the top digit.  Workgroups of <= 8 waves keep one
    // 11-bit histogram per wave (fewer colliding LDS atomics), merged
    // afterwards; larger workgroups use the shared histogram's full width.
    constexpr bool kWaveHist = kWaves <= 8;
    constexpr int D1 = kWaveHist ? 11 : digit_bits<BINS>();
    constexpr int S1 = 32 - D1;
    uint32_t* wh = kWaveHist ? dyn + wid * kWaveHistBins : s.hist;
    if (kWaveHist)
      for (int i = lane; i < kWaveHistBins; i += kWave) wh[i] = 0;
    clear_hist<NT>(s);
    __syncthreads();
    for_chunks<NT, E>(src, n, vec, [&](int64_t, const uint32_t (&key)[E], int nv) {
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (e < nv) atomicAdd(&wh[key[e] >> S1], 1u);
    });
    __syncthreads();
    if (kWaveHist) {
      for (int b = threadIdx.x; b < kWaveHistBins; b += NT) {
        uint32_t c = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) c += dyn[w * kWaveHistBins + b];
        s.hist[b] = c;
      }
      __syncthreads();
    }
    select_bin<NT>(s, (uint32_t)k, parity);
    parity ^= 1;
    const uint32_t bin1 = s.sel[0];
    const uint32_t above1 = s.sel[1];
    uint32_t* cand_keys = dyn;                      // the per-wave histograms are dead now
    uint32_t* cand_cols = dyn + kCandPairs;
    uint32_t m;                                     // keys in bin1
    {
      // Pass 2: keys above bin1 go straight out; bin1's keys become candidates
      // (stored while they fit; their count decides the path afterwards).
      uint32_t gbase = 0, cbase = 0;
      for_chunks<NT, E>(src, n, vec, [&](int64_t c0, const uint32_t (&key)[E], int nv) {
        uint32_t cg = 0, cq = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          cg += (e < nv && (key[e] >> S1) > bin1) ? 1u : 0u;
          cq += (e < nv && (key[e] >> S1) == bin1) ? 1u : 0u;
        }
        uint32_t total;
        const uint32_t pre = block_scan<NT>(cg | (cq << 16), s, parity, total);
        parity ^= 1;
        uint32_t g = gbase + (pre & 0xffffu), q = cbase + (pre >> 16);
        const int64_t col0 = lo + c0 + (int64_t)E * threadIdx.x;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if (e >= nv) continue;
          const uint32_t b = key[e] >> S1;
          if (b > bin1) {
            if (g < (uint32_t)k) out[g] = (int32_t)(col0 + e);
            ++g;
          } else if (b == bin1) {
            if (q < (uint32_t)kCandPairs) {
              cand_keys[q] = key[e];
              cand_cols[q] = (uint32_t)(col0 + e);
            }
            ++q;
          }
        }
        gbase += total & 0xffffu;
        cbase += total >> 16;
      });
      m = cbase;
      __syncthreads();
    }
    uint32_t u_t, need_ties;
    if (m <= (uint32_t)kCandPairs) {
      // candidates back into registers, consecutive per thread
      constexpr int E2 = kCandPairs / NT;
      uint32_t key[E2], cols[E2];
      const int first = E2 * threadIdx.x;
      const int nv = max(0, min(E2, (int)m - first));
#pragma unroll
      for (int e = 0; e < E2; ++e) {
        key[e] = (e < nv) ? cand_keys[first + e] : 0u;
        cols[e] = (e < nv) ? cand_cols[first + e] : 0u;
      }
      refine_regs<NT>(s, key, nv, 0u, S1, bin1, (uint32_t)k - above1, parity, u_t, need_ties);
      uint32_t gr = 0, tr = 0;
      emit_regs<NT, true>(s, key, cols, 0, nv, 0u, u_t, need_ties, false, S1, bin1, out, above1, k,
                          parity, gr, tr);
      return;
    }
    // more than 8192 keys in the threshold bin: the remaining levels re-read the row
    constexpr int D = digit_bits<BINS>();
    uint32_t need = (uint32_t)k - above1, prefix = bin1;
    for (int shift = S1; shift > 0;) {
      const int nsh = shift > D ? shift - D : 0;
      const uint32_t dmask = (1u << (shift - nsh)) - 1u;
      for (int64_t c0 = 0; c0 < n; c0 += C) {
        uint32_t key[E];
        const int nv = load_keys<E>(src + c0, n - c0, vec, key);
        hist_level(s, key, nv, 0u, shift, prefix, nsh, dmask);
      }
      __syncthreads();
      select_bin<NT>(s, need, parity);
      parity ^= 1;
      need -= s.sel[1];
      prefix = (prefix << (shift - nsh)) | s.sel[0];
      shift = nsh;
    }
    u_t = prefix;
    need_ties = need;
    uint32_t gr = 0, tr = 0;
    for (int64_t c0 = 0; c0 < n; c0 += C) {
      uint32_t key[E];
      const int nv = load_keys<E>(src + c0, n - c0, vec, key);
      emit_regs<NT, false>(s, key, key, lo + c0 + (int64_t)E * threadIdx.x, nv, 0u, u_t, need_ties,
                           true, S1, bin1, out, above1, k, parity, gr, tr);
    }
  }
}

template <int NT, int E, int BINS, bool kLong>
__global__ __launch_bounds__(NT) void topk_kernel(const float* __restrict__ logits, int64_t ld,
                                                  const int32_t* __restrict__ ks,
                                                  const int32_t* __restrict__ ke, int k,
                                                  int32_t* __restrict__ out_idx) {
  __shared__ Shared<BINS> s;
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];   // long rows only
  topk_row<NT, E, BINS, kLong>(s, dyn, logits, ld, blockIdx.x, ks, ke, k, out_idx);
}

// ---------------------------------------------------------------------------
// Long rows split over workgroups, in two launches.  With few long rows, one
// workgroup per row leaves most CUs idle and the longest row sets the time.
//
// Parts: part p of row r -- columns [lo + p*P, lo + (p+1)*P), P = kPartKeys,
// held in registers by one 512-thread workgroup -- picks a threshold t_p with
// about 1.5 k * (part length / row length) + 32 of its keys at or above it
// (one histogram level over the part's own key range) and writes those (key,
// column) pairs in column order to its region of the workspace, with its
// count and t_p (0 when it kept every key).  A row of at most P keys is
// selected whole by its part 0.
//
// Merge, one 1024-thread workgroup per split row: every key of the row at or
// above T = max_p t_p was kept by its part, so when at least k kept keys are
// >= T the row's top-k lies among the kept pairs and is their top-k.
// Otherwise -- a region overflowed, more pairs than the merge holds, or parts
// so unlike that fewer than k kept keys reach T -- it selects over the whole
// row as the one-workgroup kernel does.  The launch boundary makes the parts'
// pairs visible to the merge (no fences or counters inside either kernel:
// with one launch and a device counter, the per-workgroup L2 write-backs
// serialized within each XCD).
//
// Workspace: headers [rows][parts] (count, t_p or 0, a lower bound of the kept
// keys, the part's largest key), then pair regions [rows][parts][kPartPairs]
// (key, column); nothing needs initializing.
constexpr int kPartThreads = 512;
constexpr int kPartE = 16;
constexpr int64_t kPartKeys = (int64_t)kPartThreads * kPartE;
constexpr int kSplitMaxParts = 64;
constexpr int kSplitMaxRows = 512;
constexpr int kPartPairs = 4096;
constexpr int kMergeThreads = 1024;
constexpr int kMergePairs = 8192;       // 8 per thread of the merging workgroup

__host__ __device__ constexpr int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

struct SplitWs {
  uint4* hdr;
  uint2* pairs;
  __host__ __device__ SplitWs(void* base, int64_t rows, int parts) {
    uint8_t* b = static_cast<uint8_t*>(base);
    hdr = reinterpret_cast<uint4*>(b);
    pairs = reinterpret_cast<uint2*>(b + align256(rows * parts * 16));
  }
  static int64_t bytes(int64_t rows, int parts) {
    return align256(rows * parts * 16) + rows * parts * (int64_t)kPartPairs * 8;
  }
};

__device__ __forceinline__ int64_t visible_len(const int32_t* __restrict__ ks,
                                               const int32_t* __restrict__ ke, int64_t r,
                                               int64_t ld, int64_t& lo) {
  lo = ks ? max((int64_t)ks[r], (int64_t)0) : 0;
  const int64_t hi = min((int64_t)ke[r], ld);
  return hi > lo ? hi - lo : 0;
}

template <int NT, int E, int BINS>
__global__ __launch_bounds__(NT) void topk_part_kernel(const float* __restrict__ logits,
                                                       int64_t ld, const int32_t* __restrict__ ks,
                                                       const int32_t* __restrict__ ke, int k,
                                                       int32_t* __restrict__ out_idx,
                                                       void* __restrict__ workspace, int64_t rows,
                                                       int parts) {
  constexpr int kWaves = NT / kWave;
  constexpr int64_t C = (int64_t)NT * E;
  static_assert(C == kPartKeys, "part size");
  __shared__ Shared<BINS> s;
  __shared__ int item_rp[2];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  // Work items are listed row by row, row r holding max(1, its part count)
  // of them, and workgroup i takes item i: the grid (rows x parts, an upper
  // bound) ends with the workgroups that have no item, so those do not delay
  // the dispatch of live ones.  Wave 0 finds (row, part) from a prefix over
  // the rows' visible lengths.
  if (wid == 0) {
    const int64_t item = blockIdx.x;
    int64_t base = 0;
    int found_r = -1, found_p = 0;
    for (int64_t r0 = 0; r0 < rows; r0 += kWave) {
      const int64_t rr = r0 + lane;
      uint32_t cnt = 0;
      if (rr < rows) {
        int64_t lo_r;
        const int64_t n_r = visible_len(ks, ke, rr, ld, lo_r);
        cnt = (uint32_t)max((int64_t)1, (n_r + C - 1) / C);
      }
      const uint32_t incl = wave_incl_scan(cnt);
      const int64_t first = base + incl - cnt;
      const bool mine = rr < rows && item >= first && item < first + cnt;
      const uint64_t m = __ballot(mine);
      if (m) {                                    // wave-uniform
        const int src = (int)__builtin_ctzll(m);
        found_r = __builtin_amdgcn_readlane((int)rr, src);
        found_p = __builtin_amdgcn_readlane((int)(item - first), src);
        break;
      }
      base += __builtin_amdgcn_readlane((int)incl, 63);
    }
    if (lane == 0) {
      item_rp[0] = found_r;
      item_rp[1] = found_p;
    }
  }
  __syncthreads();
  if (item_rp[0] < 0) return;                     // past the last item
  const int64_t r = item_rp[0];
  const int p = item_rp[1];
  int64_t lo;
  const int64_t n = visible_len(ks, ke, r, ld, lo);
  const int nparts = (int)((n + C - 1) / C);
  if (nparts <= 1) {
    topk_row<NT, E, BINS, false>(s, nullptr, logits, ld, r, ks, ke, k, out_idx);
    return;
  }
  const SplitWs ws(workspace, rows, parts);
  int parity = 0;
  const int64_t c0 = (int64_t)p * C;
  const int64_t np = min(C, n - c0);
  const float* src = logits + r * ld + lo + c0;
  const bool vec = (reinterpret_cast<uintptr_t>(src) & 15) == 0;
  uint32_t key[E];
  const int nv = load_keys<E>(src, np, vec, key);
  clear_hist<NT>(s);
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (e < nv) {
      kmin = min(kmin, key[e]);
      kmax = max(kmax, key[e]);
    }
  kmin = ~wave_umax(~kmin);
  kmax = wave_umax(kmax);
  if (lane == 0) {
    s.wave_tot[1][wid] = kmin;
    s.wave_tot[1][kMaxWaves + wid] = kmax;
  }
  __syncthreads();
  kmin = ~wave_umax(lane < kWaves ? ~s.wave_tot[1][lane & 15] : 0u);
  kmax = wave_umax(lane < kWaves ? s.wave_tot[1][kMaxWaves + (lane & 15)] : 0u);
  const int64_t want = min(np, ((int64_t)3 * k * np) / (2 * n) + 32);
  uint32_t t_p = kmin;                            // keep all (one distinct key, or want = np)
  const uint32_t range = kmax - kmin;
  if (range != 0 && want < np) {
    const int L = 32 - __clz(range);
    constexpr int D = digit_bits<BINS>();
    const int nsh = L > D ? L - D : 0;
    // the estimate histograms every other key (half the LDS atomics; the
    // merge's checks keep the result exact whatever the estimate)
    constexpr int EH = E / 2;
    uint32_t half[EH];
#pragma unroll
    for (int e = 0; e < EH; ++e) half[e] = key[2 * e];
    const int nvh = (nv + 1) / 2;
    hist_first(s, half, nvh, kmin, nsh);
    __syncthreads();
    select_bin<NT>(s, (uint32_t)max((int64_t)1, want / 2), parity);   // its scan writes wave_tot[0]
    parity ^= 1;
    t_p = kmin + (s.sel[0] << nsh);               // lower edge of the want-th key's bin
  }
  uint32_t cnt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) cnt += (e < nv && key[e] >= t_p) ? 1u : 0u;
  uint32_t kept;
  uint32_t pos = block_scan<NT>(cnt, s, parity, kept);
  if (kept <= (uint32_t)kPartPairs) {
    uint2* region = ws.pairs + (r * parts + p) * (int64_t)kPartPairs;
    const uint32_t col0 = (uint32_t)(lo + c0 + (int64_t)E * threadIdx.x);
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (e < nv && key[e] >= t_p) region[pos++] = make_uint2(key[e], col0 + (uint32_t)e);
  }
  if (threadIdx.x == 0) ws.hdr[r * parts + p] = make_uint4(kept, t_p == kmin ? 0u : t_p, t_p, kmax);
}

template <int NT, int E, int BINS>
__global__ __launch_bounds__(NT) void topk_part_merge_kernel(const float* __restrict__ logits,
                                                             int64_t ld,
                                                             const int32_t* __restrict__ ks,
                                                             const int32_t* __restrict__ ke, int k,
                                                             int32_t* __restrict__ out_idx,
                                                             const void* __restrict__ workspace,
                                                             int64_t rows, int parts) {
  constexpr int E2 = kMergePairs / NT;
  __shared__ Shared<BINS> s;
  __shared__ uint32_t pbase[kSplitMaxParts + 1];
  __shared__ uint32_t mstat[5];           // T, total, overflow / spill, key bounds
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
  const int64_t r = blockIdx.x;
  int64_t lo;
  const int64_t n = visible_len(ks, ke, r, ld, lo);
  const int nparts = (int)((n + kPartKeys - 1) / kPartKeys);
  if (nparts <= 1) return;                      // selected by the part kernel
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const SplitWs ws(const_cast<void*>(workspace), rows, parts);
  int parity = 0;
  if (threadIdx.x == 0) s.ccount = 0;
  clear_hist<NT>(s);
  // Pairs are loaded before the headers arrive: part q gets NT / P2 threads
  // (P2 = the part count rounded up to a power of two, >= 2), thread j of
  // them slots j*E2 .. j*E2 + E2-1 of the part's region -- at most 4096
  // slots, so always inside the region; the headers then tell which slots
  // hold pairs.  A part that kept more than its share of slots sends the
  // merge to a dense reload.
  int p2 = 2;
  while (p2 < nparts) p2 <<= 1;
  const int tpp = NT / p2;
  const int sq = (int)threadIdx.x / tpp;
  const uint32_t sbase = (uint32_t)(((int)threadIdx.x % tpp) * E2);
  uint32_t mkey[E2], mcol[E2];
  if (sq < nparts) {
    const uint2* reg = ws.pairs + (r * parts + sq) * (int64_t)kPartPairs + sbase;
#pragma unroll
    for (int e = 0; e < E2; ++e) {
      const uint2 pr = reg[e];
      mkey[e] = pr.x;
      mcol[e] = pr.y;
    }
  }
  if (wid == 0) {
    const uint4 h = lane < nparts ? ws.hdr[r * parts + lane] : make_uint4(0u, 0u, 0xffffffffu, 0u);
    const uint32_t inc = wave_incl_scan(h.x);
    const uint32_t tstar = wave_umax(h.y);
    const uint32_t klo = ~wave_umax(~h.z);      // every kept key lies in [klo, khi]
    const uint32_t khi = wave_umax(h.w);
    const bool over = __ballot(h.x > (uint32_t)kPartPairs) != 0;
    const bool spill = __ballot(h.x > (uint32_t)(tpp * E2)) != 0;
    if (lane < nparts) pbase[lane + 1] = inc;
    if (lane == 0) {
      pbase[0] = 0;
      mstat[0] = tstar;
      mstat[1] = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
      mstat[2] = (over ? 1u : 0u) | (spill ? 2u : 0u);
      mstat[3] = klo;
      mstat[4] = khi;
    }
  }
  __syncthreads();
  const uint32_t tstar = mstat[0], total = mstat[1];
  const bool spill = (mstat[2] & 2u) != 0;
  if (!(mstat[2] & 1u) && (!spill || total <= (uint32_t)kMergePairs)) {
    // each thread's valid slots are a prefix of its E2, and only those are candidates
    int nv2;
    if (!spill) {
      const uint32_t kq = sq < nparts ? pbase[sq + 1] - pbase[sq] : 0u;
      nv2 = (int)min((uint32_t)E2, kq - min(kq, sbase));
    } else {
      // dense: thread t takes the kept pairs E2*t .. E2*t + E2-1 of all parts in order
      const uint32_t first = (uint32_t)(E2 * threadIdx.x);
      nv2 = (int)min((uint32_t)E2, total - min(total, first));
      int q = 0;                                 // part holding pair `first`
      for (int step = kSplitMaxParts / 2; step > 0; step >>= 1)
        if (q + step < nparts && pbase[q + step] <= first) q += step;
#pragma unroll
      for (int e = 0; e < E2; ++e) {
        const uint32_t i = first + (uint32_t)e;
        if (e < nv2) {
          while (pbase[q + 1] <= i) ++q;
          const uint2 pr = ws.pairs[(r * parts + q) * (int64_t)kPartPairs + (i - pbase[q])];
          mkey[e] = pr.x;
          mcol[e] = pr.y;
        }
      }
    }
    uint32_t reach = 0;
#pragma unroll
    for (int e = 0; e < E2; ++e) {
      if (e < nv2) {
        reach += mkey[e] >= tstar ? 1u : 0u;
      } else {
        mkey[e] = 0u;
        mcol[e] = 0xffffffffu;
      }
    }
    uint32_t reach_all;
    (void)block_scan<NT>(reach, s, parity, reach_all);
    parity ^= 1;
    if (reach_all >= (uint32_t)k) {
      // at least k kept keys reach T, so the row's top-k is the top-k of the kept pairs
      __syncthreads();                            // wave_tot reads done before select_pairs
      // the kept pairs are all valid: their count and key bounds come from the
      // headers, so the selection skips its own range and count pass
      const uint32_t okmask = (1u << nv2) - 1u;
      select_pairs_ranged<NT, kFewMerge>(s, mkey, mcol, okmask, nv2, k, out_idx + r * (int64_t)k,
                                         parity, mstat[3], mstat[4], total);
      return;
    }
  }
  __syncthreads();                                // shared state is reused below
  topk_row<NT, E, BINS, true>(s, dyn, logits, ld, r, ks, ke, k, out_idx);
}

// ---------------------------------------------------------------------------
// Merge of per-rank top-k lists (the exchange step of context-parallel
// decode, P3 "SparseAttnIndexerKpool": dcp_rank / dcp_world_size /
// cp_kv_cache_interleave_size).  Rank s holds the sequence's positions in
// runs of `interleave`, dealt round-robin; its local position l is global
// position (l / I) * I * R + s * I + l % I.  Row r's candidates are the
// R * k_in (value, local position) entries of all ranks (position -1 = empty
// slot); the result is the k best by value descending, then global position
// ascending -- the same set the unsharded top-k would give.
//
// One workgroup per row, E candidates per thread in rank-major order.  Empty
// slots become (the smallest valid key, column 0xffffffff): they rank below
// every real candidate and are never needed when at least k are valid.  The
// threshold is found as an exact (key, column) pair: either the few-candidate
// ranking of the first radix level's bin, or the key radix select followed by
// a radix select over the columns of the keys tied at the threshold (lowest
// first); the output takes every candidate at or above that pair, in
// candidate order (deterministic).
template <int NT, int E>
__global__ __launch_bounds__(NT) void topk_merge_kernel(const float* __restrict__ values,
                                                        const int32_t* __restrict__ indices,
                                                        int world, int k_in, int64_t rows,
                                                        int interleave, int k,
                                                        int32_t* __restrict__ out_idx) {
  constexpr int BINS = 2048;
  __shared__ Shared<BINS> s;
  const int64_t r = blockIdx.x;
  int32_t* out = out_idx + r * k;
  const int ncand = world * k_in;
  const int parity = 0;
  if (threadIdx.x == 0) s.ccount = 0;           // read only after later barriers
  clear_hist<NT>(s);                            // first read after the barriers below

  // candidates c = E*t + e: rank c / k_in, slot c % k_in
  const int first = E * (int)threadIdx.x;
  const int nv = max(0, min(E, ncand - first));
  uint32_t key[E], col[E];
  uint32_t okmask = 0;
  {
    int sh = first / k_in, j = first - sh * k_in;
    const int64_t span = (int64_t)interleave * world;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      key[e] = 0;
      col[e] = 0xffffffffu;
      if (e < nv) {
        const int64_t off = ((int64_t)sh * rows + r) * k_in + j;
        const int li = indices[off];
        if (li >= 0) {
          okmask |= 1u << e;
          key[e] = f32_key(__float_as_uint(values[off]));
          col[e] = (uint32_t)((li / interleave) * span + (int64_t)sh * interleave + li % interleave);
        }
      }
      if (++j == k_in) {
        j = 0;
        ++sh;
      }
    }
  }
  select_pairs<NT, kFewMerge>(s, key, col, okmask, nv, k, out, parity);
}

// Kernels that take more than the default dynamic LDS need the attribute set
// once per device.  The per-device flags are atomics (release after the set,
// acquire before skipping it), so concurrent first calls from several host
// threads are well defined: at worst two of them both set the attribute.
constexpr int kAttrDevices = 64;

hipError_t allow_dyn_lds(const void* kernel, int bytes, std::atomic<bool>* flags) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool tracked = dev >= 0 && dev < kAttrDevices;
  if (tracked && flags[dev].load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  if (tracked) flags[dev].store(true, std::memory_order_release);
  return hipSuccess;
}

// One set of flags per kernel instantiation.
template <int NT, int E, int BINS>
std::atomic<bool>* attr_flags() {
  static std::atomic<bool> flags[kAttrDevices];
  return flags;
}

template <int NT, int E, int BINS>
hipError_t launch_cfg(const float* logits, int64_t rows, int64_t ld, const int32_t* ks,
                      const int32_t* ke, int k, int32_t* out_idx, hipStream_t stream) {
  const bool long_rows = ld > (int64_t)NT * E;
  // 64 KB: candidate pairs, or first the per-wave histograms (<= 8 x 8 KB)
  const size_t dyn = long_rows ? (size_t)kCandPairs * 2 * sizeof(uint32_t) : 0;
  if (!long_rows) {
    hipLaunchKernelGGL((topk_kernel<NT, E, BINS, false>), dim3((unsigned)rows), dim3(NT), 0, stream,
                       logits, ld, ks, ke, k, out_idx);
    return hipGetLastError();
  }
  hipError_t e = allow_dyn_lds(reinterpret_cast<const void*>(topk_kernel<NT, E, BINS, true>),
                               (int)dyn, attr_flags<NT, E, BINS>());
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((topk_kernel<NT, E, BINS, true>), dim3((unsigned)rows), dim3(NT), dyn, stream,
                     logits, ld, ks, ke, k, out_idx);
  return hipGetLastError();
}

// Rows split over workgroups: few rows (fewer than the 512 that fill the chip
// with one workgroup each), rows longer than one part, and at most
// kSplitMaxParts parts per row.
int split_parts(int64_t rows, int64_t ld) {
  if (rows < 1 || rows >= kSplitMaxRows || ld <= kPartKeys) return 0;
  const int64_t parts = (ld + kPartKeys - 1) / kPartKeys;
  return parts <= kSplitMaxParts ? (int)parts : 0;
}

}  // namespace

// Scratch of the allocation-free entry point (launch_topk_noalloc): the split
// top-k's workspace as a file-scope device array of kNoAllocScratchBytes.  Each
// device that loads the library holds its own copy until the process ends.  In
// host code `scratch` names a host-side stand-in, never the device memory: the
// device address is taken once per device, with that device current, from
// hipGetSymbolAddress and kept in g_scratch_ptr; only that address is passed to
// kernels.
__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
std::atomic<void*> g_scratch_ptr[kAttrDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch` (set up on the first call per device).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kAttrDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}
}  // namespace

int64_t topk_workspace_bytes(int64_t rows, int64_t ld) {
  const int parts = split_parts(rows, ld);
  return parts ? SplitWs::bytes(rows, parts) : 0;
}

hipError_t launch_topk_ws(const float* logits, int64_t rows, int64_t ld, const int32_t* ks,
                          const int32_t* ke, int k, int32_t* out_idx, void* workspace,
                          hipStream_t stream) {
  const int parts = split_parts(rows, ld);
  if (!parts) return launch_topk(logits, rows, ld, ks, ke, k, out_idx, stream);
  // the merge's whole-row fallback uses the long-row path's 64 KB of LDS
  constexpr size_t dyn = (size_t)kCandPairs * 2 * sizeof(uint32_t);
  static std::atomic<bool> merge_attr[kAttrDevices];
  const auto merge = topk_part_merge_kernel<kMergeThreads, 16, 2048>;
  hipError_t e = allow_dyn_lds(reinterpret_cast<const void*>(merge), (int)dyn, merge_attr);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((topk_part_kernel<kPartThreads, kPartE, 2048>),
                     dim3((unsigned)(parts * rows)), dim3(kPartThreads), 0, stream, logits, ld, ks,
                     ke, k, out_idx, workspace, rows, parts);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge, dim3((unsigned)rows), dim3(kMergeThreads), dyn, stream, logits, ld, ks,
                     ke, k, out_idx, static_cast<const void*>(workspace), rows, parts);
  return hipGetLastError();
}

hipError_t launch_topk_merge(const float* values, const int32_t* indices, int world, int k_in,
                             int64_t rows, int interleave, int k, int32_t* out_idx,
                             hipStream_t stream) {
  const int ncand = world * k_in;
#define MXIDX_MERGE(e)                                                                         \
  hipLaunchKernelGGL((topk_merge_kernel<1024, e>), dim3((unsigned)rows), dim3(1024), 0, stream, \
                     values, indices, world, k_in, rows, interleave, k, out_idx)
  // at most 8192 candidates per row (checked by the ABI): 8 per thread keeps the
  // candidates, their columns and the tie keys in registers
  if (ncand <= 4 * 1024)
    MXIDX_MERGE(4);
  else
    MXIDX_MERGE(8);
#undef MXIDX_MERGE
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int64_t rows, int64_t ld, const int32_t* ks,
                       const int32_t* ke, int k, int32_t* out_idx, hipStream_t stream) {
  // Few rows: 1024 threads per row (the row's latency is the step's); many
  // rows: 512 threads, two rows per CU.  Wider digits (fewer levels) lose:
  // the per-level histogram clear and scan grow with the bin count.
  // Keys per thread: the smallest size that holds a full row in one pass.
  if (rows < 512) {
    if (ld <= 4 * 1024) return launch_cfg<1024, 4, 2048>(logits, rows, ld, ks, ke, k, out_idx, stream);
    if (ld <= 8 * 1024) return launch_cfg<1024, 8, 2048>(logits, rows, ld, ks, ke, k, out_idx, stream);
    return launch_cfg<1024, 16, 2048>(logits, rows, ld, ks, ke, k, out_idx, stream);
  }
  if (ld <= 8 * 512) return launch_cfg<512, 8, 2048>(logits, rows, ld, ks, ke, k, out_idx, stream);
  return launch_cfg<512, 16, 2048>(logits, rows, ld, ks, ke, k, out_idx, stream);
}

hipError_t launch_topk_noalloc(const float* logits, int64_t rows, int64_t ld, const int32_t* ks,
                               const int32_t* ke, int k, int32_t* out_idx, hipStream_t stream) {
  if (topk_workspace_bytes(rows, ld) > kNoAllocScratchBytes) return hipErrorInvalidValue;
  void* ws = nullptr;
  if (split_parts(rows, ld)) {
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return e;
  }
  // the split workspace needs no initialization: every header and pair the
  // merge reads is written by the part launch of the same call
  return launch_topk_ws(logits, rows, ld, ks, ke, k, out_idx, ws, stream);
}

}  // namespace mxidx
