// One-workgroup keep-set selection of a row (ROWS mode; [EVICT] "KV-cache
// eviction strategies", section 4.2 H2O and section 4.1 StreamingLLM): the
// first `sinks` and last `window` positions of a row are always kept; among
// the middle positions the k = budget - |forced| largest scores are kept,
// equal scores resolved toward the lower position.  The row's workgroup
//   1. radix-selects on order-preserving uint32 keys (11 + 11 + 10 bit
//      digits, histograms in LDS with integer atomics) the k-th largest middle
//      key tau and how many of the keys equal to tau are still needed;
//   2. keeps, in an ordered pass over the row in tiles, the forced positions,
//      the keys above tau and the first needed ties in position order,
//      writing the kept positions ascending (block-wide exclusive scans give
//      the slots).
// Shared by the selection kernels and by the H2O step, which settles a list
// that must shed more than one slot inside its own workgroup.
#pragma once

#include "device_common.hpp"

namespace kvsel {

namespace {

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

}  // namespace

}  // namespace kvsel
