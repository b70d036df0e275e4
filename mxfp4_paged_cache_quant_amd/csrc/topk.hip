// Per-row top-k over the visible columns [ks, ke) (top_k_per_row of P3
// "SparseAttnIndexerKpool"; exact sets, as P2 "Validation" tests them).
//
// Ranking: value descending, then column ascending; -0.0 == +0.0.  The output
// holds the min(k, n) selected columns (in column order within each selection
// stage) followed by -1.
//
// Radix select on order-preserving 32-bit keys, one 1024-thread workgroup per
// row, histograms in LDS:
//   level 1: bits 31..21 (2048 bins), level 2: bits 20..10 (2048 bins),
//   level 3: bits 9..0 (1024 bins).
// Each level finds the bin in which the running count from the top crosses
// the number still needed; after level 3 the exact k-th key T is known, and a
// final ordered pass takes every key > T plus the lowest-column keys == T.
// Order-dependent writes use block-wide prefix sums (never atomics), so the
// output is deterministic.
//
// Where the row lives during the passes:
//   * n <= 16384: the keys are cached in LDS on the first (only) HBM read;
//   * longer rows: a second HBM pass writes the level-1 winners (keys above
//     the threshold bin) directly and compacts the threshold bin's candidates
//     (key, column) into LDS; if the bin holds more than 8192 candidates, the
//     later levels re-read the row from memory and filter by prefix.
#include "common.hpp"
#include "launch.hpp"

namespace mxidx {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kCacheKeys = 16384;            // 64 KB of LDS
constexpr int kCandPairs = kCacheKeys / 2;   // (key, column) pairs in the same space

struct TopkShared {
  uint32_t hist[2048];
  uint32_t buf[kCacheKeys];   // cached keys, or candidate keys [0, 8192) + columns [8192, 16384)
  uint32_t wave_sums[kWaves];
  int sel[2];                 // selected bin, count strictly above it
};

__device__ __forceinline__ uint32_t key_of(const float* row, int64_t c) {
  return f32_key(__float_as_uint(row[c]));
}

// Exclusive prefix sum over the workgroup (thread order); also returns the total.
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* wave_sums, uint32_t& total) {
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wave_sums[wid] = x;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const uint32_t s = wave_sums[i];
    before += (i < wid) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + x - v;
}

// Finds the bin b (scanning from the top) where the count of keys in bins > b
// is < need and the count in bins >= b is >= need.  Requires need >= 1 and a
// histogram total >= need.  Result in s.sel[0] (bin), s.sel[1] (count above).
__device__ void select_bin(TopkShared& s, int nbins, uint32_t need) {
  const int t = threadIdx.x;
  const int b0 = nbins - 1 - 2 * t;
  const int b1 = b0 - 1;
  const uint32_t c0 = (b0 >= 0) ? s.hist[b0] : 0u;
  const uint32_t c1 = (b1 >= 0) ? s.hist[b1] : 0u;
  uint32_t total;
  const uint32_t before = block_scan(c0 + c1, s.wave_sums, total);
  if (b0 >= 0 && before < need && before + c0 >= need) {
    s.sel[0] = b0;
    s.sel[1] = (int)before;
  }
  if (b1 >= 0 && before + c0 < need && before + c0 + c1 >= need) {
    s.sel[0] = b1;
    s.sel[1] = (int)(before + c0);
  }
  __syncthreads();
}

__device__ __forceinline__ void clear_hist(TopkShared& s) {
  for (int i = threadIdx.x; i < 2048; i += kThreads) s.hist[i] = 0;
  __syncthreads();
}

// Candidate sources.  get(i, key, col) returns false when item i is not part
// of the current candidate set.
struct CachedRow {     // all n keys of the row in LDS, column = lo + i
  const uint32_t* keys;
  int64_t lo;
  __device__ bool get(int64_t i, uint32_t& key, int64_t& col) const {
    key = keys[i];
    col = lo + i;
    return true;
  }
};
struct CandPairs {     // compacted (key, column) pairs of the level-1 bin, in column order
  const uint32_t* keys;
  const uint32_t* cols;
  __device__ bool get(int64_t i, uint32_t& key, int64_t& col) const {
    key = keys[i];
    col = (int64_t)cols[i];
    return true;
  }
};
struct GlobalRow {     // re-read from memory, keeping keys of the level-1 bin
  const float* row;
  int64_t lo;
  uint32_t bin1;
  __device__ bool get(int64_t i, uint32_t& key, int64_t& col) const {
    key = key_of(row, lo + i);
    col = lo + i;
    return (key >> 21) == bin1;
  }
};

// Levels 2 and 3 on a candidate source; returns the exact threshold key and
// the number of keys equal to it that must still be taken.
template <typename Src>
__device__ void refine(TopkShared& s, const Src& src, int64_t count, uint32_t bin1, uint32_t need2,
                       uint32_t& thresh, uint32_t& need_ties) {
  clear_hist(s);
  for (int64_t i = threadIdx.x; i < count; i += kThreads) {
    uint32_t key;
    int64_t col;
    if (src.get(i, key, col) && (key >> 21) == bin1) atomicAdd(&s.hist[(key >> 10) & 2047u], 1u);
  }
  __syncthreads();
  select_bin(s, 2048, need2);
  const uint32_t bin2 = (uint32_t)s.sel[0];
  const uint32_t need3 = need2 - (uint32_t)s.sel[1];
  const uint32_t prefix = (bin1 << 11) | bin2;
  __syncthreads();
  clear_hist(s);
  for (int64_t i = threadIdx.x; i < count; i += kThreads) {
    uint32_t key;
    int64_t col;
    if (src.get(i, key, col) && (key >> 10) == prefix) atomicAdd(&s.hist[key & 1023u], 1u);
  }
  __syncthreads();
  select_bin(s, 1024, need3);
  thresh = (prefix << 10) | (uint32_t)s.sel[0];
  need_ties = need3 - (uint32_t)s.sel[1];
  __syncthreads();
}

// Ordered final pass: writes every candidate with key > thresh (restricted to
// the level-1 bin when only_bin1) and the first need_ties candidates with
// key == thresh, at out[base + rank in candidate order].
template <typename Src>
__device__ void emit(TopkShared& s, const Src& src, int64_t count, uint32_t thresh,
                     uint32_t need_ties, bool only_bin1, uint32_t bin1, int32_t* out,
                     uint32_t base, int k) {
  uint32_t gt_base = 0, tie_base = 0;
  for (int64_t c0 = 0; c0 < count; c0 += kThreads) {
    const int64_t i = c0 + threadIdx.x;
    uint32_t key = 0;
    int64_t col = 0;
    bool gt = false, tie = false;
    if (i < count && src.get(i, key, col) && (!only_bin1 || (key >> 21) == bin1)) {
      gt = key > thresh;
      tie = key == thresh;
    }
    uint32_t total;
    const uint32_t pre = block_scan((gt ? 1u : 0u) | (tie ? 0x10000u : 0u), s.wave_sums, total);
    const uint32_t gt_pre = gt_base + (pre & 0xffffu);
    const uint32_t tie_pre = tie_base + (pre >> 16);
    const uint32_t pos = base + gt_pre + min(tie_pre, need_ties);
    if ((gt || (tie && tie_pre < need_ties)) && pos < (uint32_t)k) out[pos] = (int32_t)col;
    gt_base += total & 0xffffu;
    tie_base += total >> 16;
  }
}

__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ logits, int64_t ld,
                                                        const int32_t* __restrict__ ks,
                                                        const int32_t* __restrict__ ke, int k,
                                                        int32_t* __restrict__ out_idx) {
  __shared__ TopkShared s;
  const int64_t r = blockIdx.x;
  const float* row = logits + r * ld;
  int32_t* out = out_idx + r * (int64_t)k;
  const int64_t lo = ks ? max((int64_t)ks[r], (int64_t)0) : 0;
  const int64_t hi = min((int64_t)ke[r], ld);
  const int64_t n = hi > lo ? hi - lo : 0;

  if (n <= k) {
    for (int i = threadIdx.x; i < k; i += kThreads) out[i] = (i < n) ? (int32_t)(lo + i) : -1;
    return;
  }

  // Level 1 (bits 31..21), first read of the row.
  clear_hist(s);
  const bool cached = n <= kCacheKeys;
  for (int64_t i = threadIdx.x; i < n; i += kThreads) {
    const uint32_t key = key_of(row, lo + i);
    if (cached) s.buf[i] = key;
    atomicAdd(&s.hist[key >> 21], 1u);
  }
  __syncthreads();
  select_bin(s, 2048, (uint32_t)k);
  const uint32_t bin1 = (uint32_t)s.sel[0];
  const uint32_t above1 = (uint32_t)s.sel[1];
  const uint32_t m = s.hist[bin1];
  __syncthreads();

  uint32_t thresh, need_ties;
  if (cached) {
    const CachedRow src{s.buf, lo};
    refine(s, src, n, bin1, (uint32_t)k - above1, thresh, need_ties);
    emit(s, src, n, thresh, need_ties, false, bin1, out, 0u, k);
    return;
  }

  // Long row: second read writes the keys above bin1 and compacts bin1.
  const bool fits = m <= (uint32_t)kCandPairs;
  uint32_t* cand_keys = s.buf;
  uint32_t* cand_cols = s.buf + kCandPairs;
  {
    uint32_t above_base = 0, cand_base = 0;
    for (int64_t c0 = 0; c0 < n; c0 += kThreads) {
      const int64_t i = c0 + threadIdx.x;
      bool gt = false, eq = false;
      uint32_t key = 0;
      if (i < n) {
        key = key_of(row, lo + i);
        gt = (key >> 21) > bin1;
        eq = (key >> 21) == bin1;
      }
      uint32_t total;
      const uint32_t pre = block_scan((gt ? 1u : 0u) | (eq ? 0x10000u : 0u), s.wave_sums, total);
      const uint32_t pos = above_base + (pre & 0xffffu);
      if (gt && pos < (uint32_t)k) out[pos] = (int32_t)(lo + i);
      if (eq && fits) {
        const uint32_t p = min(cand_base + (pre >> 16), (uint32_t)(kCandPairs - 1));
        cand_keys[p] = key;
        cand_cols[p] = (uint32_t)(lo + i);
      }
      above_base += total & 0xffffu;
      cand_base += total >> 16;
    }
    __syncthreads();
  }
  if (fits) {
    const CandPairs src{cand_keys, cand_cols};
    refine(s, src, (int64_t)m, bin1, (uint32_t)k - above1, thresh, need_ties);
    emit(s, src, (int64_t)m, thresh, need_ties, true, bin1, out, above1, k);
  } else {
    const GlobalRow src{row, lo, bin1};
    refine(s, src, n, bin1, (uint32_t)k - above1, thresh, need_ties);
    emit(s, src, n, thresh, need_ties, true, bin1, out, above1, k);
  }
}

}  // namespace

hipError_t launch_topk(const float* logits, int64_t rows, int64_t ld, const int32_t* ks,
                       const int32_t* ke, int k, int32_t* out_idx, hipStream_t stream) {
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)rows), dim3(kThreads), 0, stream, logits, ld, ks,
                     ke, k, out_idx);
  return hipGetLastError();
}

}  // namespace mxidx
