// Keep-set selection: sinks + heavy hitters + recent window per row, and the
// cross-request top-K on per-request percentiles.
//
// ROWS mode ([EVICT] "KV-cache eviction strategies", §4.2 H2O and §4.1
// StreamingLLM): the first `sinks` and last `window` positions of a row are
// always kept; among the middle positions the k = budget - |forced| largest
// scores are kept, equal scores resolved toward the lower position.  One
// workgroup per row:
//   1. radix select on order-preserving uint32 keys (11 + 11 + 10 bit digits,
//      histograms in LDS with integer atomics) finds the k-th largest middle
//      key tau and how many of the keys equal to tau are still needed;
//   2. an ordered pass over the row in tiles keeps forced positions, keys
//      above tau, and the first needed ties in position order, writing the
//      kept positions ascending (block-wide exclusive scans give the slots).
// GLOBAL_PERCENTILE mode ([OFFLOAD] "Sparse attention x KV-cache offloading",
// §3.2): each row is sorted in LDS (bitonic) to rank its items; the
// percentile (rank + 1) / n becomes the exact integer key
// floor((rank + 1) * 2^43 / n), which orders and ties exactly like the
// rational for n <= 2^20; packed above the inverted global position it gives
// distinct 64-bit composites whose top-K (radix select in one workgroup)
// equals the top-K by (percentile desc, row asc, position asc).
#include <algorithm>

#include "device_common.hpp"
#include "kvsel_internal.hpp"

namespace kvsel {

namespace {

constexpr int kSelThreads = 512;     // global-percentile kernels
constexpr int kRowThreads = 1024;    // per-row select
#ifndef KVSEL_ROW_UNROLL
#define KVSEL_ROW_UNROLL 2   // same-box A/B: 128 x 8192 top-128 22.0 -> 17.0 us; 128 x ~20K at 20% 32.2 -> 31.5 us (8 was the old value)
#endif
#ifndef KVSEL_SUB_HIST
#define KVSEL_SUB_HIST 4
#endif
constexpr int kRowUnroll = KVSEL_ROW_UNROLL;  // independent loads in flight per thread
constexpr int kSubHist = KVSEL_SUB_HIST;      // LDS sub-histograms (waves w, w+kSubHist, ... share one)

// Order-preserving map from float to uint32 (larger float -> larger key);
// -0.0 is folded onto +0.0 first.
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x == 0.f ? 0.f : x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan of one int per thread over the block of NT threads; `total`
// receives the block sum.  `ws` needs NT / 64 ints.  Every thread must call it.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* ws, int& total) {
  constexpr int kSelWaves = NT / kWave;
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  int x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) ws[w] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) {
    const int t = ws[i];
    before += i < w ? t : 0;
    all += t;
  }
  __syncthreads();
  total = all;
  return before + x - v;
}

// Given a histogram of `nb` bins (nb a multiple of NT), find digit d with
// count(bins > d) < rank <= count(bins >= d), rank >= 1.  Returns d and sets
// `above` to count(bins > d).
template <int NT>
__device__ int find_digit(const int* hist, int nb, int rank, int* ws, int* res, int& above) {
  const int per = nb / NT;
  const int tid = threadIdx.x;
  // thread t owns bins [nb - (t+1)*per, nb - t*per): scanning threads in
  // order walks the bins from the top.
  const int hi_bin = nb - tid * per;  // exclusive
  int local = 0;
  for (int i = 1; i <= per; ++i) local += hist[hi_bin - i];
  int total;
  const int before = block_exclusive_scan<NT>(local, ws, total);  // bins above my range
  int run = before;
  for (int i = 1; i <= per; ++i) {
    const int bin = hi_bin - i;
    const int c = hist[bin];
    if (run < rank && rank <= run + c) {
      res[0] = bin;
      res[1] = run;
    }
    run += c;
  }
  __syncthreads();
  above = res[1];
  const int d = res[0];
  __syncthreads();
  return d;
}

struct RowsParams {
  const float* scores;
  int64_t stride;
  const int32_t* lengths;
  const int32_t* budgets;
  int max_budget, sinks, window;
  int32_t* out_idx;
  int64_t out_stride;
  int32_t* out_count;
};

// LDS of the one-workgroup row selection.
struct RowLds {
  __attribute__((aligned(16))) int hist[kSubHist][2048];
  int ws[kRowThreads / kWave];
  int res[2];
};

// Selection of row r with budget B by one workgroup of NT threads (every
// thread calls it; NT a multiple of 256 up to kRowThreads).
template <int NT = kRowThreads>
__device__ void select_row(const RowsParams& p, int r, RowLds& sh, int B) {
  auto& hist = sh.hist;
  int* ws = sh.ws;
  int* res = sh.res;
  const int tid = threadIdx.x;
  const int n = p.lengths[r];
  const float* row = p.scores + (size_t)r * p.stride;
  int32_t* out = p.out_idx + (size_t)r * p.out_stride;
  const int lo = min(p.sinks, n);
  const int hi = max(n - p.window, 0);
  const bool keep_all = B >= n || hi <= lo;
  const int fsize = keep_all ? n : lo + (n - hi);
  const int k = keep_all ? 0 : max(0, B - fsize);
  if (k == 0) {
    // Everything, or exactly the forced positions [0, lo) and [hi, n).
    for (int j = tid; j < n; j += NT) {
      if (keep_all) out[j] = j;
      else if (j < lo) out[j] = j;
      else if (j >= hi) out[lo + (j - hi)] = j;
    }
    if (tid == 0) p.out_count[r] = fsize;
    return;
  }

  // ---- radix select of the k-th largest key among positions [lo, hi) ------
  // Each pass streams the middle with kRowUnroll independent loads in flight
  // per thread and counts digits in one of kSubHist LDS histograms.
  int* my_hist = hist[(tid / kWave) % kSubHist];
  const bool vec = (p.stride & 3) == 0 && (reinterpret_cast<uintptr_t>(p.scores) & 15) == 0;
  uint32_t prefix = 0, pmask = 0;
  int rank = k;
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = shifts[pass];
    const uint32_t dmask = (1u << widths[pass]) - 1u;
    const int nb = 1 << widths[pass];
    for (int i = tid; i < kSubHist * 2048; i += NT) (&hist[0][0])[i] = 0;
    __syncthreads();
    if (vec) {
      // 16-byte loads of aligned quads covering [lo, hi); lanes mask the edges
      const int q_lo = lo >> 2, q_hi = (hi + 3) >> 2;
      for (int q0 = q_lo + tid; q0 < q_hi; q0 += NT * kRowUnroll) {
        float4 v[kRowUnroll];
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u) {
          const int q = q0 + u * NT;
          v[u] = q < q_hi ? reinterpret_cast<const float4*>(row)[q] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u) {
          const int j = (q0 + u * NT) * 4;
          const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint32_t kk = order_key(e[c]);
            if (j + c >= lo && j + c < hi && (kk & pmask) == prefix)
              atomicAdd(&my_hist[(kk >> sh) & dmask], 1);
          }
        }
      }
    } else {
      for (int j0 = lo + tid; j0 < hi; j0 += NT * kRowUnroll) {
        float v[kRowUnroll];
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u) {
          const int j = j0 + u * NT;
          v[u] = j < hi ? row[j] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kRowUnroll; ++u) {
          const uint32_t kk = order_key(v[u]);
          if (j0 + u * NT < hi && (kk & pmask) == prefix) atomicAdd(&my_hist[(kk >> sh) & dmask], 1);
        }
      }
    }
    __syncthreads();
    for (int i = tid; i < nb; i += NT) {
      int c = 0;
#pragma unroll
      for (int h = 0; h < kSubHist; ++h) c += hist[h][i];
      hist[0][i] = c;
    }
    __syncthreads();
    int above;
    const int d = find_digit<NT>(hist[0], nb, rank, ws, res, above);
    rank -= above;
    prefix |= (uint32_t)d << sh;
    pmask |= dmask << sh;
  }
  const uint32_t tau = prefix;
  const int ties_needed = rank;  // keys equal to tau to keep, lowest positions first

  // ---- ordered output pass -------------------------------------------------
  int tie_base = 0, out_base = 0;
  for (int t0 = 0; t0 < n; t0 += NT * 4) {
    const int j0 = t0 + tid * 4;
    float sv[4];
    if (vec && j0 + 3 < n) {
      const float4 v4 = reinterpret_cast<const float4*>(row)[j0 >> 2];
      sv[0] = v4.x; sv[1] = v4.y; sv[2] = v4.z; sv[3] = v4.w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[i] = (j0 + i < n) ? row[j0 + i] : 0.f;
    }
    int eq[4], keep[4];
    int n_eq = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + i;
      const bool mid = j >= lo && j < hi;
      const uint32_t kk = (j < n && mid) ? order_key(sv[i]) : 0u;
      eq[i] = (j < n && mid && kk == tau) ? 1 : 0;
      keep[i] = (j < n) ? ((!mid) || kk > tau ? 1 : 0) : 0;
      n_eq += eq[i];
    }
    int eq_total;
    const int eq_before = tie_base + block_exclusive_scan<NT>(n_eq, ws, eq_total);
    int run = eq_before, n_keep = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (eq[i]) {
        keep[i] = run < ties_needed ? 1 : 0;
        ++run;
      }
      n_keep += keep[i];
    }
    int keep_total;
    int pos = out_base + block_exclusive_scan<NT>(n_keep, ws, keep_total);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (keep[i]) out[pos++] = j0 + i;
    tie_base += eq_total;
    out_base += keep_total;
  }
  if (tid == 0) p.out_count[r] = out_base;
}

// Rows of at most kRowThreads positions: one position per thread, its key
// held in a register through the three radix passes (LDS histograms only,
// no re-reads of the row), then the ordered output by block scans.  Same
// result as the radix selection over global memory.
constexpr int kSmallRow = kRowThreads;

__device__ void select_row_small(const RowsParams& p, int r, RowLds& sh, int B) {
  int* hist = sh.hist[0];
  int* ws = sh.ws;
  int* res = sh.res;
  const int tid = threadIdx.x;
  const int n = p.lengths[r];
  const float* row = p.scores + (size_t)r * p.stride;
  int32_t* out = p.out_idx + (size_t)r * p.out_stride;
  const int lo = min(p.sinks, n);
  const int hi = max(n - p.window, 0);
  const bool keep_all = B >= n || hi <= lo;
  const int fsize = keep_all ? n : lo + (n - hi);
  const int k = keep_all ? 0 : max(0, B - fsize);
  const bool mid = tid >= lo && tid < hi;
  int keep;
  if (keep_all || k == 0) {
    keep = tid < n && (keep_all || !mid) ? 1 : 0;
  } else {
    const uint32_t key = mid ? order_key(row[tid]) : 0u;
    uint32_t prefix = 0, pmask = 0;
    int rank = k;
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
      const int shf = shifts[pass];
      const uint32_t dmask = (1u << widths[pass]) - 1u;
      const int nb = 1 << widths[pass];
      for (int i = tid; i < nb; i += kRowThreads) hist[i] = 0;
      __syncthreads();
      if (mid && (key & pmask) == prefix) atomicAdd(&hist[(key >> shf) & dmask], 1);
      __syncthreads();
      int above;
      const int d = find_digit<kRowThreads>(hist, nb, rank, ws, res, above);
      rank -= above;
      prefix |= (uint32_t)d << shf;
      pmask |= dmask << shf;
    }
    // keys above tau are kept; of the keys equal to tau, the `rank` lowest
    // positions
    const bool eq = mid && key == prefix;
    int eq_total;
    const int eq_before = block_exclusive_scan<kRowThreads>(eq ? 1 : 0, ws, eq_total);
    keep = tid < n && (!mid || key > prefix || (eq && eq_before < rank)) ? 1 : 0;
  }
  int total;
  const int pos = block_exclusive_scan<kRowThreads>(keep, ws, total);
  if (keep) out[pos] = tid;
  if (tid == 0) p.out_count[r] = total;
}

__device__ __forceinline__ int row_budget(const RowsParams& p, int r) {
  return p.budgets ? p.budgets[r] : p.max_budget;
}

__global__ __launch_bounds__(kRowThreads) void select_rows_kernel(RowsParams p) {
  __shared__ RowLds sh;
  if (p.lengths[blockIdx.x] <= kSmallRow) select_row_small(p, blockIdx.x, sh, row_budget(p, blockIdx.x));
  else select_row(p, blockIdx.x, sh, row_budget(p, blockIdx.x));
}

// ---- ROWS mode, split over workgroups (long rows, small budgets) ---------
// One workgroup per row leaves most of the chip idle when a few hundred rows
// are each tens of thousands of positions long, and reading every row twice
// (a histogram pass, then a compaction pass) doubles the traffic.  Such rows
// are selected in three launches that read the scores once:
//   1. sample kernel (one workgroup per row): the middle keys of one 16-
//      position line in every 16 give an estimate of the row's distribution;
//      a lower bound tau_lo is put a few standard deviations below the
//      sample's estimate of the cut (the k-th largest middle key);
//   2. compaction kernel (one wave per 1024-position segment): the middle
//      positions whose key is at least tau_lo are stored with their keys, in
//      position order, per segment (ballots give each lane its slots);
//   3. final kernel (one workgroup per row): if at least k positions were
//      stored, the cut is among them: each thread loads a run of consecutive
//      stored entries into registers, a radix select over them finds tau and
//      the ties still needed, and one scan places the kept positions in order
//      between the forced ranges.
// The bound only decides how much is stored, never the result: a row whose
// stored positions are fewer than k (the sample over-estimated the cut) or
// more than the final kernel holds (many ties, or a sample that
// under-estimated it) is selected from its scores by the one-workgroup
// algorithm inside the final kernel.  Results are identical either way.
// Digits here are 8 bits, counted in 16 copies of a 256-bin histogram (lane
// mod 16 picks the copy): the keys near a cut crowd into few bins, and the
// copies bound the lanes of one instruction that hit the same LDS word.
constexpr int kLine = 16;              // positions per sampled line (64 bytes)
constexpr int kSampleEvery = 16;       // one line in this many is sampled
constexpr int kUnit = 8;               // sampled positions per thread and load (half a line)
constexpr int kSampleThreads = kRowThreads;
constexpr int kSampleRegUnits = 2;     // sample units per thread kept in registers
#ifndef KVSEL_OUT_SEG
#define KVSEL_OUT_SEG 1024
#endif
#ifndef KVSEL_COMPACT_WAVES
#define KVSEL_COMPACT_WAVES 4
#endif
constexpr int kOutSeg = KVSEL_OUT_SEG;  // compaction segment: one wave, kOutSeg / 256 float4 per lane
constexpr int kCapSeg = kOutSeg;       // entries stored per segment: all of it, so no overflow
constexpr int kCompactWaves = KVSEL_COMPACT_WAVES;  // segments per compaction workgroup
constexpr int kFinThreads = 512;
constexpr int kFinPer = 32;            // stored entries per thread in the final kernel
constexpr int kFinEnt = kFinPer * kFinThreads;  // stored entries the final kernel holds
constexpr int kFinSegs = 1024;         // compaction segments per row the split path handles
constexpr int kHCopies = 16;           // histogram copies
constexpr int kHStride = 257;          // words per copy: equal bins of copies in distinct banks
#ifndef KVSEL_SPLIT_MIN_LEN
#define KVSEL_SPLIT_MIN_LEN 16384
#endif
#ifndef KVSEL_SPLIT_MAX_ROWS
#define KVSEL_SPLIT_MAX_ROWS 2048
#endif
constexpr int kSplitMinLen = KVSEL_SPLIT_MIN_LEN;    // split rows at least this long ...
constexpr int kSplitMaxRows = KVSEL_SPLIT_MAX_ROWS;  // ... when there are at most this many rows ...
constexpr int kSplitMaxFrac = 8;                     // ... budgets keep at most 1/8 of a row ...
constexpr int kSplitMaxK = 6144;                     // ... and at most this many positions (the
                                                     // stored ones must fit the final kernel)

struct RowPlan {
  int n, lo, hi, k, fsize;
  bool keep_all;
};

__device__ __forceinline__ RowPlan row_plan(const RowsParams& p, int r) {
  RowPlan q;
  q.n = p.lengths[r];
  const int B = p.budgets ? p.budgets[r] : p.max_budget;
  q.lo = min(p.sinks, q.n);
  q.hi = max(q.n - p.window, 0);
  q.keep_all = B >= q.n || q.hi <= q.lo;
  q.fsize = q.keep_all ? q.n : q.lo + (q.n - q.hi);
  q.k = q.keep_all ? 0 : max(0, B - q.fsize);
  return q;
}

struct SplitParams {
  RowsParams rp;
  uint32_t* tau;     // [rows]: lower bound of the stored keys (top 16 bits; the rest 0)
  int* counts;       // [rows][n_oseg]: stored entries per segment
  uint2* slots;      // [rows][n_oseg][kCapSeg]: (position, key) of middle positions with key >= tau
  int n_oseg;        // segments of kOutSeg positions per row
  int max_len;       // positions below it lie inside every row (stride >= max_len)
};

// Buffer resource over positions [0, n_valid) of a row: loads past it
// return 0 instead of reading memory, so a thread's loads need no branch and
// can all be in flight at once, from one offset register each.  Rows 16-byte
// aligned: the range is rounded up to a whole quad, which stays inside the
// row (aligned rows are at least round_up(length, 4) floats apart).  Word 3
// selects 32-bit data, which untyped loads need to be valid.
template <bool kVec>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const float* row, int n_valid) {
  const int words = kVec ? ((n_valid + 3) & ~3) : n_valid;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row), (short)0, words * 4, 0x00020000);
}

// Positions j0 .. j0+3 of a row through its buffer resource (j0 >= 0, a
// multiple of 4 when kVec; positions past the resource read as 0).
template <bool kVec>
__device__ __forceinline__ float4 load4(__amdgpu_buffer_rsrc_t rs, int j0) {
  if (kVec) return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, j0 * 4, 0, 0));
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (j0 + i) * 4, 0, 0));
  return make_float4(v[0], v[1], v[2], v[3]);
}

// Sample unit u of a row: half u % 2 of sampled line u / 2, i.e. positions
// (u/2)*256 + (u%2)*8 .. +7 (the last unit when u >= n_units, whose keys
// unit_keys then drops).
template <bool kVec>
__device__ __forceinline__ void unit_load(__amdgpu_buffer_rsrc_t rs, int u, int n_units, float4 (&v)[kUnit / 4]) {
  const int uc = min(u, n_units - 1);
  const int j0 = (uc >> 1) * kLine * kSampleEvery + (uc & 1) * kUnit;
#pragma unroll
  for (int c4 = 0; c4 < kUnit / 4; ++c4) v[c4] = load4<kVec>(rs, j0 + c4 * 4);
}

// Top 16 bits of the keys of a sample unit; 0 marks a position outside the
// middle or a unit past the row (a key whose top 16 bits are 0, a NaN with
// those bits set, is left out of the sample, which only changes the
// estimate).
__device__ __forceinline__ void unit_keys(const float4 (&v)[kUnit / 4], int u, int n_units, int lo, int hi,
                                          uint32_t (&kk)[kUnit]) {
  const int j0 = (u >> 1) * kLine * kSampleEvery + (u & 1) * kUnit;
#pragma unroll
  for (int c4 = 0; c4 < kUnit / 4; ++c4) {
    const float e[4] = {v[c4].x, v[c4].y, v[c4].z, v[c4].w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = j0 + c4 * 4 + c;
      kk[c4 * 4 + c] = (u < n_units && j >= lo && j < hi) ? order_key(e[c]) >> 16 : 0u;
    }
  }
}

// LDS of the 8-bit radix steps: two sets of 16-copy histograms (pass p adds
// into set p & 1 while the other is cleared for pass p + 1), per-wave sums
// of the 256 bins and the step's result, each doubled the same way, so one
// step needs three barriers.
struct DigitLds {
  int h[2][kHCopies * kHStride];
  int wsum[2][256 / kWave];
  int res[2][2];
  int total;
};

__device__ __forceinline__ void hist_add(int* h, uint32_t bin) {
  atomicAdd(&h[(threadIdx.x & (kHCopies - 1)) * kHStride + bin], 1);
}

// Clears set 0 and the total before the first pass (a barrier must follow).
template <int NT>
__device__ __forceinline__ void digit_init(DigitLds& L) {
  for (int i = threadIdx.x; i < kHCopies * kHStride; i += NT) L.h[0][i] = 0;
  if (threadIdx.x == 0) L.total = 0;
}

// One digit step, called by every thread (NT >= 256) after the barrier that
// follows pass p's hist_add calls into set p & 1: threads t < 256 sum bin
// 255 - t over the copies (so that scanning threads in order walks the bins
// from the top) while set (p + 1) & 1 is cleared; the digit d with
// count(digits > d) < rank <= count(digits >= d) is then found with one
// wave scan and one exchange of wave sums.  rank >= 1 and at most the
// pass's total.  Returns d and sets above = count(digits > d).
template <int NT>
__device__ int digit_step(DigitLds& L, int p, int rank, int& above) {
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave, cur = p & 1;
  const int* h = L.h[cur];
  int c = 0;
  if (tid < 256) {
#pragma unroll
    for (int k = 0; k < kHCopies; ++k) c += h[k * kHStride + (255 - tid)];
  }
  for (int i = tid; i < kHCopies * kHStride; i += NT) L.h[cur ^ 1][i] = 0;
  int x = c;
  if (tid < 256) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(x, off, kWave);
      if (lane >= off) x += y;
    }
    if (lane == kWave - 1) L.wsum[cur][w] = x;
  }
  __syncthreads();
  if (tid < 256) {
    int before = x - c;
#pragma unroll
    for (int i = 0; i < 256 / kWave; ++i) before += i < w ? L.wsum[cur][i] : 0;
    if (before < rank && rank <= before + c) {
      L.res[cur][0] = 255 - tid;
      L.res[cur][1] = before;
    }
  }
  __syncthreads();
  above = L.res[cur][1];
  return L.res[cur][0];
}

// tau_lo of row r: with m sampled middle keys out of n_mid, the cut's
// expected rank in the sample is k_s = k m / n_mid.  The count of the row's
// k largest keys that fall in the sample has variance at most kLine * k_s
// (binomial over lines, each line holding up to kLine of them when they come
// in runs, as max-pooled scores do; runs longer than the sampling period are
// sampled systematically), so the sample's k_lo-th largest key,
// k_lo = k_s + 4 sqrt(kLine k_s) + 4, is below the cut unless that count is
// 4 standard deviations above its mean.  tau_lo is that key truncated to its
// top 16 bits (two 8-bit digits; the sample keeps only those bits); 0 (store
// every middle position) when the sample holds fewer than k_lo keys.
template <bool kVec>
__global__ __launch_bounds__(kSampleThreads) void select_split_sample(SplitParams sp) {
  constexpr int NT = kSampleThreads;
  __shared__ DigitLds L;
  const RowsParams& p = sp.rp;
  const int r = blockIdx.x, tid = threadIdx.x;
  // The register units' loads go out before the row's plan is read (their
  // range is every row's [0, max_len); keys outside the middle are dropped)
  const auto rs = row_rsrc<kVec>(p.scores + (size_t)r * p.stride, sp.max_len);
  const int n_units_max = 2 * ((sp.max_len + kLine * kSampleEvery - 1) / (kLine * kSampleEvery));
  float4 raw[kSampleRegUnits][kUnit / 4];
#pragma unroll
  for (int it = 0; it < kSampleRegUnits; ++it) unit_load<kVec>(rs, tid + it * NT, n_units_max, raw[it]);
  __builtin_amdgcn_sched_barrier(0);
  const RowPlan q = row_plan(p, r);
  if (q.k == 0) return;
  const int n_units = 2 * ((q.hi + kLine * kSampleEvery - 1) / (kLine * kSampleEvery));  // below hi
  digit_init<NT>(L);
  __syncthreads();
  uint32_t kr[kSampleRegUnits][kUnit];
  int m = 0;
#pragma unroll
  for (int it = 0; it < kSampleRegUnits; ++it) {
    unit_keys(raw[it], tid + it * NT, n_units, q.lo, q.hi, kr[it]);
#pragma unroll
    for (int c = 0; c < kUnit; ++c)
      if (kr[it][c]) {
        hist_add(L.h[0], kr[it][c] >> 8);
        ++m;
      }
  }
  for (int u = tid + kSampleRegUnits * NT; u < n_units; u += NT) {   // units past the register ones
    float4 v[kUnit / 4];
    uint32_t kk[kUnit];
    unit_load<kVec>(rs, u, n_units, v);
    unit_keys(v, u, n_units, q.lo, q.hi, kk);
#pragma unroll
    for (int c = 0; c < kUnit; ++c)
      if (kk[c]) {
        hist_add(L.h[0], kk[c] >> 8);
        ++m;
      }
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) m += __shfl_xor(m, off, kWave);
  if (tid % kWave == 0 && m) atomicAdd(&L.total, m);
  __syncthreads();
  const int m_all = L.total;
  const double k_s = (double)q.k * m_all / (double)(q.hi - q.lo);
  const int k_lo = (int)ceil(k_s + 4.0 * sqrt((double)kLine * k_s) + 4.0);
  if (k_lo > m_all) {
    if (tid == 0) sp.tau[r] = 0u;
    return;
  }
  int above;
  const int d1 = digit_step<NT>(L, 0, k_lo, above);
#pragma unroll
  for (int it = 0; it < kSampleRegUnits; ++it)
#pragma unroll
    for (int c = 0; c < kUnit; ++c)
      if (kr[it][c] && (int)(kr[it][c] >> 8) == d1) hist_add(L.h[1], kr[it][c] & 0xFFu);
  for (int u = tid + kSampleRegUnits * NT; u < n_units; u += NT) {
    float4 v[kUnit / 4];
    uint32_t kk[kUnit];
    unit_load<kVec>(rs, u, n_units, v);
    unit_keys(v, u, n_units, q.lo, q.hi, kk);
#pragma unroll
    for (int c = 0; c < kUnit; ++c)
      if (kk[c] && (int)(kk[c] >> 8) == d1) hist_add(L.h[1], kk[c] & 0xFFu);
  }
  __syncthreads();
  const int d2 = digit_step<NT>(L, 1, k_lo - above, above);
  if (tid == 0) sp.tau[r] = ((uint32_t)d1 << 24) | ((uint32_t)d2 << 16);
}

// Segments of row r (kOutSeg positions each, one wave per segment): the
// middle positions whose key is at least the row's tau_lo are stored in
// position order with their keys; the segment's count goes to `counts`.  A
// lane holds positions j0 .. j0+3 of each 256-position step, so in position
// order an entry follows every entry of the lanes below it in the same step:
// one ballot per position within the quad gives each lane its slot.
template <bool kVec>
__global__ __launch_bounds__(kWave * kCompactWaves) void select_split_compact(SplitParams sp) {
  constexpr int IT = kOutSeg / (4 * kWave);
  const RowsParams& p = sp.rp;
  const int r = blockIdx.y, s = blockIdx.x * kCompactWaves + threadIdx.x / kWave, lane = threadIdx.x % kWave;
  if (s >= sp.n_oseg) return;
  const int sb = s * kOutSeg;
  // The segment's loads go out before the row's plan is read (their range
  // is every row's [0, max_len); positions outside the middle are masked).
  const auto rs = row_rsrc<kVec>(p.scores + (size_t)r * p.stride, min(sb + kOutSeg, sp.max_len));
  float4 v[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) v[it] = load4<kVec>(rs, sb + it * 4 * kWave + lane * 4);
  __builtin_amdgcn_sched_barrier(0);   // every load is issued before the first is used
  const RowPlan q = row_plan(p, r);
  if (q.k == 0) return;
  const int j_lo = max(sb, q.lo), j_hi = min(sb + kOutSeg, q.hi);
  int* cnt = sp.counts + (size_t)r * sp.n_oseg + s;
  if (j_lo >= j_hi) {
    if (lane == 0) *cnt = 0;
    return;
  }
  const uint32_t tau = sp.tau[r];
  uint2* slot = sp.slots + ((size_t)r * sp.n_oseg + s) * kCapSeg;
  int base = 0;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int j0 = sb + it * 4 * kWave + lane * 4;
    const float e[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
    uint32_t kk[4];
    bool f[4];
    int below = 0, step = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      kk[c] = order_key(e[c]);
      f[c] = j0 + c >= j_lo && j0 + c < j_hi && kk[c] >= tau;
      const uint64_t b = __ballot(f[c]);
      below += __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
      step += __popcll(b);
    }
    int pos = base + below;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (f[c]) slot[pos++] = make_uint2((uint32_t)(j0 + c), kk[c]);
    base += step;
  }
  if (lane == 0) *cnt = base;
}

// Segment of flat entry f: the s with pre[s] <= f < pre[s + 1].
__device__ __forceinline__ int seg_of(const int* pre, int n_seg, int f) {
  int lo = 0, hi = n_seg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= f) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// One workgroup per row.  The stored entries, in position order, are split
// into runs of consecutive entries, one per thread, held in registers.  If
// there are at least k of them, the k-th largest middle key is among them.
// Every stored key is at least tau_lo, so the first digit is the key's top
// 16 bits above tau_lo's, capped at 255: when the cut lies below the cap,
// that one step fixes 16 bits and two 8-bit steps finish tau; otherwise four
// 8-bit steps over the whole keys follow.  One scan of (kept above tau, equal
// to tau) per thread then places every kept position between the forced
// ranges.  A row with fewer than k stored entries, or more than kFinEnt, is
// selected from its scores by the one-workgroup algorithm; the result is the
// same.
__global__ __launch_bounds__(kFinThreads) void select_split_final(SplitParams sp) {
  constexpr int NT = kFinThreads;
  __shared__ RowLds sh;
  __shared__ DigitLds L;
  __shared__ int seg_pre[kFinSegs + 1];
  const RowsParams& p = sp.rp;
  const int r = blockIdx.x, tid = threadIdx.x;
  // segment counts: thread t holds segments 2t and 2t + 1, loaded before the
  // row's plan is read (unused when the row needs no selection)
  static_assert(kFinSegs == 2 * NT, "two segments per thread");
  const int* cnt = sp.counts + (size_t)r * sp.n_oseg;
  const int c0_all = 2 * tid < sp.n_oseg ? cnt[2 * tid] : 0;
  const int c1_all = 2 * tid + 1 < sp.n_oseg ? cnt[2 * tid + 1] : 0;
  const RowPlan q = row_plan(p, r);
  const int n_seg = (q.n + kOutSeg - 1) / kOutSeg;
  if (q.k == 0) {
    select_row<NT>(p, r, sh, row_budget(p, r));
    return;
  }
  int* ws = sh.ws;
  const int c0 = 2 * tid < n_seg ? c0_all : 0, c1 = 2 * tid + 1 < n_seg ? c1_all : 0;
  int tot;
  const int pre = block_exclusive_scan<NT>(c0 + c1, ws, tot);
  if (2 * tid < n_seg) seg_pre[2 * tid] = pre;
  if (2 * tid + 1 < n_seg) seg_pre[2 * tid + 1] = pre + c0;
  if (tid == 0) seg_pre[n_seg] = tot;
  if (tot < q.k || tot > kFinEnt) {
    select_row<NT>(p, r, sh, row_budget(p, r));
    return;
  }
  __syncthreads();
  // this thread's run: entries [f_beg, f_end), one search for the first
  // segment, then a walk across the (rare) segment boundaries; every load is
  // issued before any is used
  const uint2* slots = sp.slots + (size_t)r * sp.n_oseg * kCapSeg;
  const int per = (tot + NT - 1) / NT;
  const int f_beg = min(tid * per, tot), f_end = min(f_beg + per, tot);
  uint2 e[kFinPer];
#pragma unroll
  for (int i = 0; i < kFinPer; ++i) e[i] = make_uint2(0u, 0u);
  if (f_beg < f_end) {
    int sg = seg_of(seg_pre, n_seg, f_beg);
    int cur = seg_pre[sg], nxt = seg_pre[sg + 1];
#pragma unroll
    for (int i = 0; i < kFinPer; ++i) {
      const int f = f_beg + i;
      if (f < f_end) {
        while (f >= nxt) {
          ++sg;
          cur = nxt;
          nxt = seg_pre[sg + 1];
        }
        e[i] = slots[(size_t)sg * kCapSeg + (f - cur)];
      }
    }
  }
  const int mine = f_end - f_beg;
  const uint32_t base16 = sp.tau[r] >> 16;
  digit_init<NT>(L);
  __syncthreads();
  // first step: top 16 bits relative to tau_lo's, capped at 255
#pragma unroll
  for (int i = 0; i < kFinPer; ++i)
    if (i < mine) hist_add(L.h[0], min((e[i].y >> 16) - base16, 255u));
  __syncthreads();
  int above;
  const int d0 = digit_step<NT>(L, 0, q.k, above);
  int rank = q.k - above;
  uint32_t prefix, pmask;
  int pass;
  if (d0 < 255) {
    prefix = (base16 + (uint32_t)d0) << 16;
    pmask = 0xFFFF0000u;
    pass = 2;            // bits 15..8, then 7..0
  } else {
    prefix = 0u;
    pmask = 0u;
    rank = q.k;
    pass = 0;            // bits 31..24 .. 7..0 over every key
  }
  for (int step = 1; pass < 4; ++pass, ++step) {
    const int shf = 24 - 8 * pass;
    int* h = L.h[step & 1];
#pragma unroll
    for (int i = 0; i < kFinPer; ++i)
      if (i < mine && (e[i].y & pmask) == prefix) hist_add(h, (e[i].y >> shf) & 0xFFu);
    __syncthreads();
    const int d = digit_step<NT>(L, step, rank, above);
    rank -= above;
    prefix |= (uint32_t)d << shf;
    pmask |= 0xFFu << shf;
  }
  const uint32_t tau = prefix;
  const int ties_needed = rank;        // keys equal to tau to keep, lowest positions first
  // one scan of (above tau, equal to tau) counts, 16 bits each
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < kFinPer; ++i)
    if (i < mine) {
      n_gt += e[i].y > tau;
      n_eq += e[i].y == tau;
    }
  int both;
  const int before = block_exclusive_scan<NT>(n_gt | (n_eq << 16), ws, both);
  int32_t* out = p.out_idx + (size_t)r * p.out_stride;
  for (int j = tid; j < q.lo; j += NT) out[j] = j;
  int eq_run = before >> 16;
  int pos = q.lo + (before & 0xFFFF) + min(eq_run, ties_needed);
#pragma unroll
  for (int i = 0; i < kFinPer; ++i)
    if (i < mine) {
      const uint32_t key = e[i].y;
      bool keep = key > tau;
      if (key == tau) keep = eq_run++ < ties_needed;
      if (keep) out[pos++] = (int)e[i].x;
    }
  const int kept = (both & 0xFFFF) + min(both >> 16, ties_needed);
  for (int j = q.hi + tid; j < q.n; j += NT) out[q.lo + kept + (j - q.hi)] = j;
  if (tid == 0) p.out_count[r] = q.lo + kept + (q.n - q.hi);
}

// Shapes that may split (the workspace is sized for them) and those that do.
inline bool may_split(int rows, int max_len) {
  return rows <= kSplitMaxRows && max_len >= kSplitMinLen && max_len <= kFinSegs * kOutSeg;
}
inline bool use_split(int rows, int max_len, int max_budget) {
  return may_split(rows, max_len) && (long long)max_budget * kSplitMaxFrac <= max_len &&
         max_budget <= kSplitMaxK;
}

inline size_t split_layout(int rows, int max_len, size_t* o_counts, size_t* o_slots) {
  const int n_seg = (max_len + kOutSeg - 1) / kOutSeg;
  const size_t a = ((size_t)rows * sizeof(uint32_t) + 255) & ~size_t(255);
  const size_t b = ((size_t)rows * n_seg * sizeof(int) + 255) & ~size_t(255);
  const size_t c = ((size_t)rows * n_seg * kCapSeg * sizeof(uint2) + 255) & ~size_t(255);
  if (o_counts) *o_counts = a;
  if (o_slots) *o_slots = a + b;
  return a + b + c;
}

hipError_t launch_split(const RowsParams& rp, int rows, int max_len, void* workspace, hipStream_t stream) {
  size_t o_counts, o_slots;
  split_layout(rows, max_len, &o_counts, &o_slots);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  SplitParams sp{rp, reinterpret_cast<uint32_t*>(ws), reinterpret_cast<int*>(ws + o_counts),
                 reinterpret_cast<uint2*>(ws + o_slots), (max_len + kOutSeg - 1) / kOutSeg, max_len};
  const dim3 cgrid((unsigned)((sp.n_oseg + kCompactWaves - 1) / kCompactWaves), (unsigned)rows);
  // rows 16-byte aligned: float4 loads
  if ((rp.stride & 3) == 0 && (reinterpret_cast<uintptr_t>(rp.scores) & 15) == 0) {
    hipLaunchKernelGGL(select_split_sample<true>, dim3(rows), dim3(kSampleThreads), 0, stream, sp);
    hipLaunchKernelGGL(select_split_compact<true>, cgrid, dim3(kWave * kCompactWaves), 0, stream, sp);
  } else {
    hipLaunchKernelGGL(select_split_sample<false>, dim3(rows), dim3(kSampleThreads), 0, stream, sp);
    hipLaunchKernelGGL(select_split_compact<false>, cgrid, dim3(kWave * kCompactWaves), 0, stream, sp);
  }
  hipLaunchKernelGGL(select_split_final, dim3(rows), dim3(kFinThreads), 0, stream, sp);
  return hipGetLastError();
}

// ---- GLOBAL_PERCENTILE ------------------------------------------------------
constexpr int kPctMaxLen = 8192;

struct PctParams {
  const float* scores;
  int64_t stride;
  const int32_t* lengths;
  int rows, max_len;
  uint64_t* comp;  // [rows][max_len] composites (0 = no item)
};

// Rank every item of a row by (score asc, position desc) with a bitonic sort
// of (key, inverted position) pairs in LDS; write the composite of each item.
__global__ __launch_bounds__(kSelThreads) void percentile_rank_kernel(PctParams p) {
  __shared__ uint64_t sk[kPctMaxLen];
  const int r = blockIdx.x;
  const int n = p.lengths[r];
  int m = 1;
  while (m < n) m <<= 1;
  const float* row = p.scores + (size_t)r * p.stride;
  // sort key: score key in the high 32 bits, (0xffffffff - position) low:
  // ascending order = score asc, then position desc.  Padding sorts last.
  for (int i = threadIdx.x; i < m; i += kSelThreads)
    sk[i] = i < n ? ((uint64_t)order_key(row[i]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)i)
                  : ~0ull;
  __syncthreads();
  for (int size = 2; size <= m; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < m; i += kSelThreads) {
        const int j = i ^ stride;
        if (j > i) {
          const bool up = (i & size) == 0;
          const uint64_t a = sk[i], b = sk[j];
          if ((a > b) == up) {
            sk[i] = b;
            sk[j] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  uint64_t* out = p.comp + (size_t)r * p.max_len;
  for (int rho = threadIdx.x; rho < p.max_len; rho += kSelThreads) {
    if (rho < n) {
      const uint32_t j = 0xffffffffu - (uint32_t)(sk[rho] & 0xffffffffu);
      const uint64_t key = (((uint64_t)(rho + 1)) << 43) / (uint64_t)n;
      const uint64_t g = (uint64_t)r * p.max_len + j;
      out[j] = (key << 20) | ((1ull << 20) - 1ull - g);
    }
  }
  // positions n .. max_len-1 hold no item
  for (int j = n + threadIdx.x; j < p.max_len; j += kSelThreads) out[j] = 0ull;
}

// K-th largest composite over all rows (radix select, 8 passes of 8 bits, one
// workgroup).  thr[0] receives the threshold (0 when K covers every item).
__global__ __launch_bounds__(kSelThreads) void global_threshold_kernel(const uint64_t* comp,
                                                                       int total, int K,
                                                                       uint64_t* thr) {
  __shared__ int hist[512];
  __shared__ int ws[kSelThreads / kWave];
  __shared__ int res[2];
  __shared__ int n_valid_s;
  const int tid = threadIdx.x;
  int cnt = 0;
  for (int i = tid; i < total; i += kSelThreads) cnt += comp[i] != 0ull;
  int n_valid;
  block_exclusive_scan<kSelThreads>(cnt, ws, n_valid);
  if (K >= n_valid || K <= 0) {
    if (tid == 0) thr[0] = K <= 0 ? ~0ull : 1ull;  // keep nothing / keep every item
    return;
  }
  (void)n_valid_s;
  uint64_t prefix = 0, pmask = 0;
  int rank = K;
  for (int pass = 0; pass < 8; ++pass) {
    const int sh = 56 - 8 * pass;
    for (int i = tid; i < 512; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < total; i += kSelThreads) {
      const uint64_t c = comp[i];
      if (c != 0ull && (c & pmask) == prefix) atomicAdd(&hist[(c >> sh) & 0xff], 1);
    }
    __syncthreads();
    int above;
    const int d = find_digit<kSelThreads>(hist, 512, rank, ws, res, above);
    rank -= above;
    prefix |= (uint64_t)d << sh;
    pmask |= 0xffull << sh;
  }
  if (tid == 0) thr[0] = prefix;  // composites are distinct: rank is now 1
}

__global__ __launch_bounds__(kSelThreads) void global_output_kernel(const uint64_t* comp,
                                                                    int max_len,
                                                                    const uint64_t* thr,
                                                                    int32_t* out_idx,
                                                                    int64_t out_stride,
                                                                    int32_t* out_count) {
  __shared__ int ws[kSelThreads / kWave];
  const int r = blockIdx.x;
  const uint64_t t = thr[0];
  const uint64_t* row = comp + (size_t)r * max_len;
  int32_t* out = out_idx + (size_t)r * out_stride;
  int base = 0;
  for (int t0 = 0; t0 < max_len; t0 += kSelThreads * 4) {
    const int j0 = t0 + threadIdx.x * 4;
    int keep[4], n_keep = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = j0 + i;
      keep[i] = (j < max_len && row[j] != 0ull && row[j] >= t) ? 1 : 0;
      n_keep += keep[i];
    }
    int tot;
    int pos = base + block_exclusive_scan<kSelThreads>(n_keep, ws, tot);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (keep[i]) out[pos++] = j0 + i;
    base += tot;
  }
  if (threadIdx.x == 0) out_count[r] = base;
}

// ---- GLOBAL_PERCENTILE in one launch ----------------------------------------
// The percentile keys of a row of n items are exactly 1/n, 2/n, ..., n/n,
// whatever its scores: the scores only decide which item takes which key.
// The global top K by (key desc, row asc) therefore fixes, from the lengths
// alone, how many items m_r each row keeps, and the row keeps its m_r best
// items by (score desc, position asc): those hold its m_r largest keys.
// Every workgroup (one per row) finds the K-th largest key T from the lengths
// by a 64-way search over the integer keys Q(k, n) = floor(k 2^43 / n) (exact
// and order-preserving for n <= 2^20), derives its m_r, and runs the row
// selection with budget m_r.  No workspace, no second launch.
constexpr int kPctFastRows = 4096;   // rows whose lengths the search holds in LDS

// Items of a row of n whose key Q(k, n) is >= T (T >= 1):
// Q(k, n) >= T  <=>  k >= T n / 2^43  (T n < 2^64 for T <= 2^43 + 1, n <= 2^20).
__device__ __forceinline__ long long pct_count_ge(uint64_t T, int n) {
  const uint64_t kmin = (T * (uint64_t)n + ((1ull << 43) - 1)) >> 43;
  const long long lo = kmin < 1 ? 1 : (long long)kmin;
  return lo > n ? 0 : (long long)n - lo + 1;
}

__global__ __launch_bounds__(kRowThreads) void global_percentile_rows_kernel(RowsParams p, int rows, int K) {
  __shared__ RowLds sh;
  __shared__ int len_s[kPctFastRows];
  __shared__ unsigned long long cnt_s[64];
  __shared__ unsigned long long lohi_s[2];
  const int tid = threadIdx.x, r = blockIdx.x;
  if (rows <= kWave) {
    // Up to 64 rows: one wave finds every row's share, lane i holding row
    // i's length, without a barrier; the others wait at the one below.
    __shared__ int m_s;
    if (tid < kWave) {
      const int ni = tid < rows ? p.lengths[tid] : 0;
      int total = ni;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) total += __shfl_xor(total, off, kWave);
      int mi;
      if (K <= 0) {
        mi = 0;
      } else if (K >= total) {
        mi = ni;
      } else {
        uint64_t lo = 1, hi = (1ull << 43) + 1;     // count_ge(lo) >= K > count_ge(hi)
        while (hi - lo > 1) {
          const uint64_t step = (hi - lo + 63) / 64;
          const uint64_t t = lo + (uint64_t)tid * step;
          long long cnt = 0;
          for (int i = 0; i < rows; ++i) cnt += pct_count_ge(t, __shfl(ni, i, kWave));
          const unsigned long long mask = __ballot(t < hi && cnt >= K);
          const uint64_t nlo = lo + (uint64_t)(63 - __builtin_clzll(mask)) * step;
          hi = nlo + step < hi ? nlo + step : hi;
          lo = nlo;
        }
        const int g = tid < rows ? (int)pct_count_ge(lo + 1, ni) : 0;
        const bool tie = tid < rows && pct_count_ge(lo, ni) > g;
        int gt = g;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) gt += __shfl_xor(gt, off, kWave);
        const unsigned long long tmask = __ballot(tie);
        const int before = __popcll(tmask & ((1ull << tid) - 1ull));
        mi = g + ((tie && before < K - gt) ? 1 : 0);
      }
      if (tid == r) m_s = mi;
    }
    __syncthreads();
    const int m = m_s;
    if (p.lengths[r] <= kSmallRow) select_row_small(p, r, sh, m);
    else select_row(p, r, sh, m);
    return;
  }
  for (int i = tid; i < rows; i += kRowThreads) len_s[i] = p.lengths[i];
  if (tid < 64) cnt_s[tid] = 0;
  __syncthreads();
  long long part = 0;
  for (int i = tid; i < rows; i += kRowThreads) part += len_s[i];
  if (part) atomicAdd(&cnt_s[0], (unsigned long long)part);
  __syncthreads();
  const long long total = (long long)cnt_s[0];
  __syncthreads();
  const int n = len_s[r];
  int m;
  if (K <= 0) {
    m = 0;
  } else if (K >= total) {
    m = n;
  } else {
    // count_ge(lo) >= K > count_ge(hi); each round tests 64 keys and keeps
    // the sub-range where the count crosses K
    uint64_t lo = 1, hi = (1ull << 43) + 1;
    const int c = tid & 63;
    while (hi - lo > 1) {
      const uint64_t step = (hi - lo + 63) / 64;
      if (tid < 64) cnt_s[tid] = 0;
      __syncthreads();
      const uint64_t t = lo + (uint64_t)c * step;
      long long q = 0;
      if (t < hi)
        for (int i = tid >> 6; i < rows; i += kRowThreads / 64) q += pct_count_ge(t, len_s[i]);
      if (q) atomicAdd(&cnt_s[c], (unsigned long long)q);
      __syncthreads();
      if (tid < kWave) {
        // the counts fall with the key: the candidates still holding K form
        // a prefix, and the highest lane of it gives the new range
        const bool ok = lo + (uint64_t)tid * step < hi && (long long)cnt_s[tid] >= K;
        const unsigned long long mask = __ballot(ok);
        const int best = 63 - __builtin_clzll(mask);     // lane 0 always qualifies
        if (tid == 0) {
          const uint64_t nlo = lo + (uint64_t)best * step;
          lohi_s[0] = nlo;
          lohi_s[1] = nlo + step < hi ? nlo + step : hi;
        }
      }
      __syncthreads();
      lo = lohi_s[0];
      hi = lohi_s[1];
    }
    // T = lo: every row keeps its keys > T, and the key equal to T (at most
    // one per row) goes to the lowest rows until K is reached
    if (tid < 2) cnt_s[tid] = 0;
    __syncthreads();
    long long gt = 0, ties_before = 0;
    for (int i = tid; i < rows; i += kRowThreads) {
      const long long g = pct_count_ge(lo + 1, len_s[i]);
      gt += g;
      if (i < r && pct_count_ge(lo, len_s[i]) > g) ++ties_before;
    }
    if (gt) atomicAdd(&cnt_s[0], (unsigned long long)gt);
    if (ties_before) atomicAdd(&cnt_s[1], (unsigned long long)ties_before);
    __syncthreads();
    const long long ties_needed = K - (long long)cnt_s[0];
    const long long g_r = pct_count_ge(lo + 1, n);
    const bool tie_r = pct_count_ge(lo, n) > g_r;
    m = (int)g_r + ((tie_r && (long long)cnt_s[1] < ties_needed) ? 1 : 0);
    __syncthreads();
  }
  if (n <= kSmallRow) select_row_small(p, r, sh, m);
  else select_row(p, r, sh, m);
}

}  // namespace

size_t select_workspace_bytes(int rows, int max_len, int mode) {
  if (mode != 1) return may_split(rows, max_len) ? split_layout(rows, max_len, nullptr, nullptr) : 0;
  return ((size_t)rows * max_len * sizeof(uint64_t) + 255 & ~size_t(255)) + 256;
}

hipError_t launch_select(const float* scores, int64_t stride, const int32_t* lengths, int rows,
                         int max_len, int sinks, int window, const int32_t* budgets,
                         int max_budget, int mode, int global_budget, int32_t* out_idx,
                         int64_t out_stride, int32_t* out_count, void* workspace,
                         hipStream_t stream) {
  if (mode == 0) {
    RowsParams rp{scores, stride, lengths, budgets, max_budget, sinks, window, out_idx, out_stride,
                  out_count};
    if (use_split(rows, max_len, max_budget)) return launch_split(rp, rows, max_len, workspace, stream);
    hipLaunchKernelGGL(select_rows_kernel, dim3(rows), dim3(kRowThreads), 0, stream, rp);
    return hipGetLastError();
  }
  if (rows <= kPctFastRows) {
    RowsParams rp{scores, stride, lengths, nullptr, 0, 0, 0, out_idx, out_stride, out_count};
    hipLaunchKernelGGL(global_percentile_rows_kernel, dim3(rows), dim3(kRowThreads), 0, stream, rp, rows,
                       global_budget);
    return hipGetLastError();
  }
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint64_t* comp = reinterpret_cast<uint64_t*>(ws);
  uint64_t* thr = reinterpret_cast<uint64_t*>(
      ws + (((size_t)rows * max_len * sizeof(uint64_t) + 255) & ~size_t(255)));
  PctParams pp{scores, stride, lengths, rows, max_len, comp};
  hipLaunchKernelGGL(percentile_rank_kernel, dim3(rows), dim3(kSelThreads), 0, stream, pp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(global_threshold_kernel, dim3(1), dim3(kSelThreads), 0, stream, comp,
                     rows * max_len, global_budget, thr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(global_output_kernel, dim3(rows), dim3(kSelThreads), 0, stream, comp,
                     max_len, thr, out_idx, out_stride, out_count);
  return hipGetLastError();
}

}  // namespace kvsel
