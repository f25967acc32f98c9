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

// Selection of row r with budget B by one workgroup of kRowThreads threads
// (every thread calls it).
__device__ void select_row(const RowsParams& p, int r, RowLds& sh, int B) {
  constexpr int NT = kRowThreads;
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
// are each tens of thousands of positions long.  Rows are then cut into
// segments:
//   1. histogram kernel: the first digit (top 11 bits of the key) of every
//      middle position, one workgroup per (segment, row), LDS histograms
//      folded into the row's global histogram with integer atomics;
//   2. compaction kernel: every workgroup finds the boundary digit d0 and
//      the rank still needed among the keys whose first digit is d0 from the
//      row's histogram, then, per 4096-position segment, stores the middle
//      positions whose first digit is above d0 (kept) or equal to it
//      (candidates) in position order with their keys, in bounded slots;
//   3. final kernel (one workgroup per row): the last two digits among the
//      candidates in LDS give tau and the ties still needed; the stored
//      positions are written out in order between the forced ranges.
// With budgets of at most 1/8 of a row the stored positions are a small
// fraction of it; a row with more stored positions than the final kernel
// holds in LDS (a boundary digit shared by many positions) is selected by
// the one-workgroup algorithm inside the final kernel.  Results are
// identical either way.
constexpr int kSegQuantum = 4096;      // segment lengths are multiples of this
#ifndef KVSEL_SEG_TARGET
#define KVSEL_SEG_TARGET 1024
#endif
constexpr int kSegTarget = KVSEL_SEG_TARGET;  // aim for about this many workgroups per kernel
constexpr int kSegThreads = 256;
constexpr int kOutSeg = 4096;          // compaction segment: 4 float4 per thread
constexpr int kCapSeg = kOutSeg;       // entries stored per compaction segment: all of it, so
                                       // keeps clustered in a few segments never overflow
constexpr int kFinEnt = 12288;         // stored entries the final kernel holds in LDS
constexpr int kFinSegs = kRowThreads;  // compaction segments per row the final kernel handles
#ifndef KVSEL_SPLIT_MIN_LEN
#define KVSEL_SPLIT_MIN_LEN 16384
#endif
#ifndef KVSEL_SPLIT_MAX_ROWS
#define KVSEL_SPLIT_MAX_ROWS 2048
#endif
constexpr int kSplitMinLen = KVSEL_SPLIT_MIN_LEN;    // split rows at least this long ...
constexpr int kSplitMaxRows = KVSEL_SPLIT_MAX_ROWS;  // ... when there are at most this many rows ...
constexpr int kSplitMaxFrac = 8;                     // ... and budgets keep at most 1/8 of a row
                                                     // (more would overflow the final kernel's LDS)

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
  uint32_t* ghist;   // [rows][2048], zero between calls
  int4* state;       // [rows]: prefix, pmask, rank after the first digit, -
  int2* counts;      // [rows][n_oseg]: stored entries, candidates
  uint2* slots;      // [rows][n_oseg][kCapSeg]: (position | candidate << 31, key) past the first digit
  int n_seg, seg_len;  // histogram passes: segments of the middle
  int n_oseg;          // count / output: segments of kOutSeg positions of the row
  bool vec;          // rows 16-byte aligned: float4 loads
};

// Loads positions j0 .. j0+3 of a row (entries outside [j_lo, j_hi) are
// returned but must be ignored by the caller).
__device__ __forceinline__ float4 load4(const float* row, bool vec, int j0, int j_lo, int j_hi) {
  if (vec) return *reinterpret_cast<const float4*>(row + j0);
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = (j0 + i >= j_lo && j0 + i < j_hi) ? row[j0 + i] : 0.f;
  return make_float4(v[0], v[1], v[2], v[3]);
}

// The first digit (top 11 bits of the order key) of every middle position of
// one segment, counted in two LDS histograms (even and odd waves) and added
// to the row's global histogram.
__global__ __launch_bounds__(kSegThreads) void select_split_hist(SplitParams sp) {
  constexpr int sh = 21;
  constexpr uint32_t dmask = 0x7FFu;
  __shared__ int hist[2][2048];
  const RowsParams& p = sp.rp;
  const int r = blockIdx.y, s = blockIdx.x, tid = threadIdx.x;
  const RowPlan q = row_plan(p, r);
  if (q.k == 0) return;
  const int j_lo = q.lo + s * sp.seg_len, j_hi = min(j_lo + sp.seg_len, q.hi);
  if (j_lo >= j_hi) return;
  for (int i = tid; i < 2 * 2048; i += kSegThreads) (&hist[0][0])[i] = 0;
  __syncthreads();
  int* my = hist[(tid / kWave) & 1];
  const float* row = p.scores + (size_t)r * p.stride;
  // aligned quads covering [j_lo, j_hi), four per thread in flight
  const int q_lo = j_lo >> 2, q_hi = (j_hi + 3) >> 2;
  constexpr int QU = 8;
  for (int q0 = q_lo + tid; q0 < q_hi; q0 += kSegThreads * QU) {
    float4 v[QU];
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      const int qq = min(q0 + u * kSegThreads, q_hi - 1);
      v[u] = load4(row, sp.vec, qq * 4, j_lo, j_hi);
    }
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      const int j = (q0 + u * kSegThreads) * 4;
      const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t kk = order_key(e[c]);
        if (q0 + u * kSegThreads < q_hi && j + c >= j_lo && j + c < j_hi) atomicAdd(&my[(kk >> sh) & dmask], 1);
      }
    }
  }
  __syncthreads();
  uint32_t* gh = sp.ghist + (size_t)r * 2048;
  for (int i = tid; i <= (int)dmask; i += kSegThreads) {
    const int c = hist[0][i] + hist[1][i];
    if (c) atomicAdd(&gh[i], (uint32_t)c);
  }
}

// The kOutSeg positions of segment s of row r, one float4 per thread and
// iteration (4 iterations), all loaded up front.
__device__ __forceinline__ void load_out_seg(const SplitParams& sp, const RowPlan& q, const float* row,
                                             int j_lo, int j_hi, float4 (&v)[kOutSeg / (4 * kSegThreads)]) {
#pragma unroll
  for (int it = 0; it < kOutSeg / (4 * kSegThreads); ++it) {
    const int j0 = j_lo + (it * kSegThreads + threadIdx.x) * 4;
    v[it] = (q.k && j0 < j_hi) ? load4(row, sp.vec, j0, j_lo, j_hi) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// Middle positions of output segment s (kOutSeg positions) that pass the
// first digit: above the row's boundary digit (kept whatever the rest of
// the selection decides) or equal to it (candidates).  They are stored in
// position order, at most kCapSeg per segment, bit 31 marking a candidate;
// the segment's (stored-or-not count, candidate count) goes to `counts`.
// Each entry carries its order key.
__global__ __launch_bounds__(kSegThreads) void select_split_compact(SplitParams sp) {
  constexpr int IT = kOutSeg / (4 * kSegThreads);
  __shared__ int ws[kSegThreads / kWave];
  __shared__ int hist[2048];
  __shared__ int res[2];
  const RowsParams& p = sp.rp;
  const int r = blockIdx.y, s = blockIdx.x, tid = threadIdx.x;
  const RowPlan q = row_plan(p, r);
  if (q.k == 0) return;
  const int sb = s * kOutSeg, sb_hi = min(sb + kOutSeg, q.n);
  int2* cnt = sp.counts + (size_t)r * sp.n_oseg + s;
  const bool empty = max(sb, q.lo) >= min(sb_hi, q.hi);
  if (empty && s != 0) {
    if (tid == 0) *cnt = make_int2(0, 0);
    return;
  }
  // The segment's scores are requested first; meanwhile every workgroup of
  // the row finds the boundary digit d0 (the first digit of the k-th largest
  // middle key) from the row's complete first-digit histogram, and the
  // row's first segment records it for the final kernel.
  const float* row = p.scores + (size_t)r * p.stride;
  float4 v[IT];
  load_out_seg(sp, q, row, sb, sb_hi, v);
  const uint32_t* gh = sp.ghist + (size_t)r * 2048;
  for (int i = tid; i < 2048; i += kSegThreads) hist[i] = (int)gh[i];
  __syncthreads();
  int above;
  const uint32_t d0 = (uint32_t)find_digit<kSegThreads>(hist, 2048, q.k, ws, res, above);
  if (s == 0 && tid == 0) sp.state[r] = make_int4((int)(d0 << 21), (int)(0x7FFu << 21), q.k - above, 0);
  if (empty) {
    if (tid == 0) *cnt = make_int2(0, 0);
    return;
  }
  uint2* slot = sp.slots + ((size_t)r * sp.n_oseg + s) * kCapSeg;
  int base = 0, n_cand = 0;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int j0 = sb + (it * kSegThreads + tid) * 4;
    const float e4[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
    int f[4], packed = 0;
    uint32_t kk[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = j0 + c;
      const bool mid = j >= q.lo && j < q.hi && j < sb_hi;
      kk[c] = order_key(e4[c]);
      const uint32_t dig = kk[c] >> 21;
      f[c] = !mid ? 0 : dig > d0 ? 1 : dig == d0 ? 2 : 0;
      packed += (f[c] != 0) + ((f[c] == 2) << 16);   // stored | candidates << 16 (both <= 4096)
    }
    int tot;
    int pos = base + (block_exclusive_scan<kSegThreads>(packed, ws, tot) & 0xFFFF);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (f[c]) {
        if (pos < kCapSeg) slot[pos] = make_uint2((uint32_t)(j0 + c) | (f[c] == 2 ? 0x80000000u : 0u), kk[c]);
        ++pos;
      }
    }
    base += tot & 0xFFFF;
    n_cand += tot >> 16;
  }
  if (tid == 0) *cnt = make_int2(base, n_cand);
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

// One workgroup per row: the row's stored entries are loaded into LDS in one
// batch; the remaining two digits are resolved among the candidates there,
// then the entries are written out in position order between the forced
// ranges.  A row whose segments overflowed their slots, or with more
// entries than LDS holds, is selected from its scores by the one-workgroup
// algorithm instead; the result is the same.
__global__ __launch_bounds__(kRowThreads) void select_split_final(SplitParams sp) {
  constexpr int NT = kRowThreads;
  constexpr int EPT = 4;                  // entries per thread and output step
  __shared__ RowLds sh;
  __shared__ uint2 ent[kFinEnt];
  __shared__ int seg_pre[kFinSegs + 1];
  const RowsParams& p = sp.rp;
  const int r = blockIdx.x, tid = threadIdx.x;
  const RowPlan q = row_plan(p, r);
  const int n_seg = (q.n + kOutSeg - 1) / kOutSeg;
  if (q.k == 0 || n_seg > kFinSegs) {
    select_row(p, r, sh, row_budget(p, r));
    return;
  }
  int* ws = sh.ws;
  const int2 c = tid < n_seg ? sp.counts[(size_t)r * sp.n_oseg + tid] : make_int2(0, 0);
  int tot;
  const int pre = block_exclusive_scan<NT>(c.x, ws, tot);
  if (tid < n_seg) seg_pre[tid] = pre;
  if (tid == 0) seg_pre[n_seg] = tot;
  if (__syncthreads_or(c.x > kCapSeg) || tot > kFinEnt) {
    select_row(p, r, sh, row_budget(p, r));
    return;
  }
  // every entry's load is issued before any is stored
  const uint2* slots = sp.slots + (size_t)r * sp.n_oseg * kCapSeg;
  constexpr int kLoads = (kFinEnt + NT - 1) / NT;
  uint2 e[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int f = tid + i * NT;
    if (f < tot) {
      const int sg = seg_of(seg_pre, n_seg, f);
      e[i] = slots[(size_t)sg * kCapSeg + (f - seg_pre[sg])];
    }
  }
#pragma unroll
  for (int i = 0; i < kLoads; ++i)
    if (tid + i * NT < tot) ent[tid + i * NT] = e[i];
  __syncthreads();
  const int4 st = sp.state[r];
  uint32_t prefix = (uint32_t)st.x, pmask = (uint32_t)st.y;
  int rank = st.z;
  int* hist = sh.hist[0];
  constexpr int kShift[2] = {10, 0};
  constexpr int kWidth[2] = {11, 10};
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int shf = kShift[pass];
    const uint32_t dmask = (1u << kWidth[pass]) - 1u;
    for (int i = tid; i < 2048; i += NT) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < tot; i += NT) {
      const uint2 v = ent[i];
      if ((v.x >> 31) && (v.y & pmask) == prefix) atomicAdd(&hist[(v.y >> shf) & dmask], 1);
    }
    __syncthreads();
    int above;
    const int d = find_digit<NT>(hist, 1 << kWidth[pass], rank, ws, sh.res, above);
    rank -= above;
    prefix |= (uint32_t)d << shf;
    pmask |= dmask << shf;
  }
  const uint32_t tau = prefix;
  const int ties_needed = rank;
  int32_t* out = p.out_idx + (size_t)r * p.out_stride;
  for (int j = tid; j < q.lo; j += NT) out[j] = j;
  int out_base = q.lo, tie_base = 0;
  for (int f0 = 0; f0 < tot; f0 += NT * EPT) {
    int keep[EPT], eq[EPT], jv[EPT], n_eq = 0;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int f = f0 + tid * EPT + i;
      keep[i] = eq[i] = jv[i] = 0;
      if (f < tot) {
        const uint2 v = ent[f];
        jv[i] = (int)(v.x & 0x7FFFFFFFu);
        if (v.x >> 31) {
          keep[i] = v.y > tau ? 1 : 0;
          eq[i] = v.y == tau ? 1 : 0;
        } else {
          keep[i] = 1;
        }
      }
      n_eq += eq[i];
    }
    int eq_total, keep_total;
    int run = tie_base + block_exclusive_scan<NT>(n_eq, ws, eq_total);
    int n_keep = 0;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      if (eq[i]) keep[i] = run++ < ties_needed ? 1 : 0;
      n_keep += keep[i];
    }
    int pos = out_base + block_exclusive_scan<NT>(n_keep, ws, keep_total);
#pragma unroll
    for (int i = 0; i < EPT; ++i)
      if (keep[i]) out[pos++] = jv[i];
    tie_base += eq_total;
    out_base += keep_total;
  }
  for (int j = q.hi + tid; j < q.n; j += NT) out[out_base + (j - q.hi)] = j;
  if (tid == 0) p.out_count[r] = out_base + (q.n - q.hi);
}

// Shapes that may split (the workspace is sized for them) and those that do.
inline bool may_split(int rows, int max_len) { return rows <= kSplitMaxRows && max_len >= kSplitMinLen; }
inline bool use_split(int rows, int max_len, int max_budget) {
  return may_split(rows, max_len) && (long long)max_budget * kSplitMaxFrac <= max_len;
}

// Segment length: a multiple of kSegQuantum giving about kSegTarget
// workgroups over all rows.
inline int split_seg_len(int rows, int max_len) {
  const int per_row = std::max(1, (kSegTarget + rows - 1) / rows);
  const int len = (max_len + per_row - 1) / per_row;
  return std::max(kSegQuantum, (len + kSegQuantum - 1) / kSegQuantum * kSegQuantum);
}

inline size_t split_layout(int rows, int max_len, size_t* o_state, size_t* o_counts, size_t* o_slots) {
  const int n_seg = (max_len + kOutSeg - 1) / kOutSeg;
  const size_t a = ((size_t)rows * 2048 * sizeof(uint32_t) + 255) & ~size_t(255);
  const size_t b = ((size_t)rows * sizeof(int4) + 255) & ~size_t(255);
  const size_t c = ((size_t)rows * n_seg * sizeof(int2) + 255) & ~size_t(255);
  const size_t d = ((size_t)rows * n_seg * kCapSeg * sizeof(uint2) + 255) & ~size_t(255);
  if (o_state) *o_state = a;
  if (o_counts) *o_counts = a + b;
  if (o_slots) *o_slots = a + b + c;
  return a + b + c + d;
}

// The global histograms must start at zero: they are cleared here once per
// call.
__global__ void select_split_zero(uint32_t* gh, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    gh[i] = 0u;
}

hipError_t launch_split(const RowsParams& rp, int rows, int max_len, void* workspace, hipStream_t stream) {
  size_t o_state, o_counts, o_slots;
  split_layout(rows, max_len, &o_state, &o_counts, &o_slots);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const int seg_len = split_seg_len(rows, max_len);
  SplitParams sp{rp, reinterpret_cast<uint32_t*>(ws), reinterpret_cast<int4*>(ws + o_state),
                 reinterpret_cast<int2*>(ws + o_counts), reinterpret_cast<uint2*>(ws + o_slots),
                 (max_len + seg_len - 1) / seg_len, seg_len, (max_len + kOutSeg - 1) / kOutSeg,
                 (rp.stride & 3) == 0 && (reinterpret_cast<uintptr_t>(rp.scores) & 15) == 0};
  const size_t nh = (size_t)rows * 2048;
  hipLaunchKernelGGL(select_split_zero, dim3((unsigned)std::min<size_t>((nh + 255) / 256, 1024)), dim3(256), 0,
                     stream, sp.ghist, nh);
  hipLaunchKernelGGL(select_split_hist, dim3(sp.n_seg, rows), dim3(kSegThreads), 0, stream, sp);
  hipLaunchKernelGGL(select_split_compact, dim3(sp.n_oseg, rows), dim3(kSegThreads), 0, stream, sp);
  hipLaunchKernelGGL(select_split_final, dim3(rows), dim3(kRowThreads), 0, stream, sp);
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
  if (mode != 1) return may_split(rows, max_len) ? split_layout(rows, max_len, nullptr, nullptr, nullptr) : 0;
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
