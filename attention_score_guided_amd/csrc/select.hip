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
#include "device_common.hpp"
#include "kvsel_internal.hpp"

namespace kvsel {

namespace {

constexpr int kSelThreads = 512;     // global-percentile kernels
constexpr int kRowThreads = 1024;    // per-row select
constexpr int kRowUnroll = 8;        // independent loads in flight per thread
constexpr int kSubHist = 4;          // LDS sub-histograms (waves w, w+4, ... share one)

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

__global__ __launch_bounds__(kRowThreads) void select_rows_kernel(RowsParams p) {
  constexpr int NT = kRowThreads;
  __shared__ int hist[kSubHist][2048];
  __shared__ int ws[NT / kWave];
  __shared__ int res[2];
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = p.lengths[r];
  const int B = p.budgets ? p.budgets[r] : p.max_budget;
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

}  // namespace

size_t select_workspace_bytes(int rows, int max_len, int mode) {
  if (mode != 1) return 0;
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
    hipLaunchKernelGGL(select_rows_kernel, dim3(rows), dim3(kRowThreads), 0, stream, rp);
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
