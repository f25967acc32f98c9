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
#include <type_traits>

#include "device_common.hpp"
#include "kvsel_internal.hpp"
#include "row_select.hpp"

namespace kvsel {

namespace {

constexpr int kSelThreads = 512;     // global-percentile kernels

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
  // Compact samples (or null): samp[r][16 m + t] is the key at position
  // 256 m + t of row r, t < 16, the positions the sample kernel reads.
  const float* samp;
  int samp_stride;
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

// Sample unit u of a compact sample row (entry i is the key at position
// 16 i): entries u*8 .. u*8+7.
__device__ __forceinline__ void unit_load_compact(__amdgpu_buffer_rsrc_t rs, int u, int n_units,
                                                  float4 (&v)[kUnit / 4]) {
  const int uc = min(u, n_units - 1);
#pragma unroll
  for (int c4 = 0; c4 < kUnit / 4; ++c4) v[c4] = load4<true>(rs, uc * kUnit + c4 * 4);
}

// Top 16 bits of the keys of a sample unit; 0 marks a position outside the
// middle or a unit past the row (a key whose top 16 bits are 0, a NaN with
// those bits set, is left out of the sample, which only changes the
// estimate).
// STRIDED: a compact unit, whose entry i is position 16 i.
template <bool STRIDED = false>
__device__ __forceinline__ void unit_keys(const float4 (&v)[kUnit / 4], int u, int n_units, int lo, int hi,
                                          uint32_t (&kk)[kUnit]) {
  const int j0 = (u >> 1) * kLine * kSampleEvery + (u & 1) * kUnit;
#pragma unroll
  for (int c4 = 0; c4 < kUnit / 4; ++c4) {
    const float e[4] = {v[c4].x, v[c4].y, v[c4].z, v[c4].w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = STRIDED ? kSampleEvery * (u * kUnit + c4 * 4 + c) : j0 + c4 * 4 + c;
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
// COMPACT: the sample is every 16th position, read from sp.samp (entry i =
// position 16 i) instead of the score rows; positions sampled one by one
// (no lines), the count has variance at most k_s, so the margin is
// 4 sqrt(k_s) + 4.
template <bool kVec, bool COMPACT = false>
__global__ __launch_bounds__(kSampleThreads) void select_split_sample(SplitParams sp) {
  constexpr int NT = kSampleThreads;
  __shared__ DigitLds L;
  const RowsParams& p = sp.rp;
  const int r = blockIdx.x, tid = threadIdx.x;
  // The register units' loads go out before the row's plan is read (their
  // range is every row's [0, max_len); keys outside the middle are dropped)
  const auto rs = COMPACT ? row_rsrc<true>(sp.samp + (size_t)r * sp.samp_stride, sp.samp_stride)
                          : row_rsrc<kVec>(p.scores + (size_t)r * p.stride, sp.max_len);
  const int n_units_max = COMPACT ? sp.samp_stride / kUnit
                                  : 2 * ((sp.max_len + kLine * kSampleEvery - 1) / (kLine * kSampleEvery));
  auto load_unit = [&](int u, int nu, float4 (&v)[kUnit / 4]) {
    if constexpr (COMPACT) unit_load_compact(rs, u, nu, v);
    else unit_load<kVec>(rs, u, nu, v);
  };
  float4 raw[kSampleRegUnits][kUnit / 4];
#pragma unroll
  for (int it = 0; it < kSampleRegUnits; ++it) load_unit(tid + it * NT, n_units_max, raw[it]);
  __builtin_amdgcn_sched_barrier(0);
  const RowPlan q = row_plan(p, r);
  if (q.k == 0) return;
  const int n_units = COMPACT ? ((q.hi + kSampleEvery - 1) / kSampleEvery + kUnit - 1) / kUnit   // below hi
                              : 2 * ((q.hi + kLine * kSampleEvery - 1) / (kLine * kSampleEvery));
  digit_init<NT>(L);
  __syncthreads();
  uint32_t kr[kSampleRegUnits][kUnit];
  int m = 0;
#pragma unroll
  for (int it = 0; it < kSampleRegUnits; ++it) {
    unit_keys<COMPACT>(raw[it], tid + it * NT, n_units, q.lo, q.hi, kr[it]);
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
    load_unit(u, n_units, v);
    unit_keys<COMPACT>(v, u, n_units, q.lo, q.hi, kk);
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
  const int k_lo = (int)ceil(k_s + 4.0 * sqrt((COMPACT ? 1.0 : (double)kLine) * k_s) + 4.0);
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
    load_unit(u, n_units, v);
    unit_keys<COMPACT>(v, u, n_units, q.lo, q.hi, kk);
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
//
// SEG is the segment size of the stored entries (kOutSeg for the
// compaction kernel).  prep(r) runs before the one-workgroup fallback of a
// row that needs its scores (every thread calls it; it may fill the row in
// sp.rp.scores).
// SPT segments per thread: rows of at most SPT * kFinThreads segments
// (seg_pre holds that many + 1).
template <int SEG, int SPT, class Prep>
__device__ void split_final_row(const SplitParams& sp, RowLds& sh, DigitLds& L, int* seg_pre, Prep&& prep) {
  constexpr int NT = kFinThreads;
  const RowsParams& p = sp.rp;
  const int r = blockIdx.x, tid = threadIdx.x;
  // segment counts: thread t holds segments SPT t .. SPT t + SPT - 1,
  // loaded before the row's plan is read (unused when the row needs no
  // selection)
  const int* cnt = sp.counts + (size_t)r * sp.n_oseg;
  int c_all[SPT];
#pragma unroll
  for (int i = 0; i < SPT; ++i) c_all[i] = SPT * tid + i < sp.n_oseg ? cnt[SPT * tid + i] : 0;
  const RowPlan q = row_plan(p, r);
  const int n_seg = (q.n + SEG - 1) / SEG;
  if (q.k == 0) {
    select_row<NT>(p, r, sh, row_budget(p, r));
    return;
  }
  int* ws = sh.ws;
  int c_sum = 0;
#pragma unroll
  for (int i = 0; i < SPT; ++i) c_sum += SPT * tid + i < n_seg ? c_all[i] : 0;
  int tot;
  int pre = block_exclusive_scan<NT>(c_sum, ws, tot);
#pragma unroll
  for (int i = 0; i < SPT; ++i)
    if (SPT * tid + i < n_seg) {
      seg_pre[SPT * tid + i] = pre;
      pre += c_all[i];
    }
  if (tid == 0) seg_pre[n_seg] = tot;
  if (tot < q.k || tot > kFinEnt) {
    prep(r);
    select_row<NT>(p, r, sh, row_budget(p, r));
    return;
  }
  __syncthreads();
  // this thread's run: entries [f_beg, f_end), one search for the first
  // segment, then a walk across the (rare) segment boundaries; every load is
  // issued before any is used
  const uint2* slots = sp.slots + (size_t)r * sp.n_oseg * SEG;
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
        e[i] = slots[(size_t)sg * SEG + (f - cur)];
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

__global__ __launch_bounds__(kFinThreads) void select_split_final(SplitParams sp) {
  __shared__ RowLds sh;
  __shared__ DigitLds L;
  __shared__ int seg_pre[kFinSegs + 1];
  static_assert(kFinSegs == 2 * kFinThreads, "two segments per thread");
  split_final_row<kOutSeg, 2>(sp, sh, L, seg_pre, [](int) {});
}

// ---- indexer top-k: the indexer's scores selected without being stored ----
// [LONGCTX] "sparse attention" experiment: a small indexer scores every
// cached key, s_j = scale * q . k_j, and each query keeps its k best keys.
// The split selection above needs the scores only three times: at the
// sampled positions (the lower bound tau_lo), once to store the keys at or
// above tau_lo, and in a row's rare fallback.  Each of these computes the
// scores it needs from K with the same MFMA chain as the indexer pass
// (K_tile (16 keys x d) . Q^T (d x the heads of a KV head), fp32
// accumulation over the k-steps in order, then * scale), so every score is
// bit-identical to what that pass would write, and the selection equals
// select_keep on those scores.  The 67 MB of scores of the 128K case are
// neither written nor read back.
struct IxkParams {
  const uint8_t* k_pages;      // [pages][H_kv][P][D] bf16 or FP8 E4M3
  const int32_t* block_table;  // [B][max_pages]
  const int32_t* seq_lens;     // [B]
  const uint8_t* q;            // [B][H_q][D] in the keys' format
  int num_kv_heads, num_q_heads, group, page_log2, max_pages, topk;
  float scale;
  float* samp;                 // [rows][samp_stride] scores at the sampled positions
  int samp_stride;             // 16 per sampled line
  int32_t* row_len;            // [rows] L_b of row r = b * H_q + h
  const uint32_t* tau;         // [rows] tau_lo
  int* counts;                 // [rows][n_oseg]
  uint2* slots;                // [rows][n_oseg][kIxkSeg]
  int n_oseg;
};

#ifndef KVSEL_IXK_QB
#define KVSEL_IXK_QB 0   // K tiles per load batch of the fused compaction (0: 8 at d = 64, 4 at d = 128)
#endif
#ifndef KVSEL_IXK_SEG
#define KVSEL_IXK_SEG 64   // 128K top-2048: 48.7 us at 64, 49.9 at 128, 51.9 at 256 (same box)
#endif
constexpr int kIxkSeg = KVSEL_IXK_SEG;   // positions per stored segment: one wave's run of a chunk
constexpr int kIxkChunk = kIxkSeg * 4;   // keys per compaction workgroup (4 waves)
constexpr int kIxkSegs = kIxkSeg >= 128 ? 2048 : 4096;   // segments per row the final pass takes (4 or 8 per thread)
constexpr int kIxkSampTiles = 4;         // sampled lines (16-key tiles) per wave
constexpr int kIxkStage = 16;            // stored entries per (wave, head) staged in LDS

// The two key formats: bf16 (one 32-channel k-step per 16-byte fragment,
// v_mfma_f32_16x16x32_bf16) and FP8 E4M3 (8-byte fragments,
// v_mfma_f32_16x16x32_fp8_fp8).  Both take D / 32 k-steps per 16 x 16 tile.
// The channels a lane feeds are those of the matching indexer pass, so
// every score is bit-identical to the one it would have written: bf16, lane
// group g gives channels u * 32 + 8 g .. + 8 to step u; FP8, lane group g
// gives channels g D / 4 + 8 u .. + 8 to step u.
template <bool F8>
using IxkFrag = std::conditional_t<F8, long, bf16x8>;

template <bool F8>
__device__ __forceinline__ f32x4 ixk_mfma(IxkFrag<F8> a, IxkFrag<F8> b, f32x4 c) {
  if constexpr (F8) return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One key or query row's fragments for lane group grp, from its first byte.
template <int D, bool F8>
__device__ __forceinline__ void ixk_row_frags(const uint8_t* row, int grp, IxkFrag<F8> (&f)[D / 32]) {
  if constexpr (F8) {
    const uint8_t* rp = row + grp * (D / 4);
#pragma unroll
    for (int v = 0; v < D / 64; ++v) {
      const uint4 w = ld16(rp + v * 16);
      f[2 * v] = (long)w.x | ((long)w.y << 32);
      f[2 * v + 1] = (long)w.z | ((long)w.w << 32);
    }
  } else {
#pragma unroll
    for (int u = 0; u < D / 32; ++u) f[u] = __builtin_bit_cast(bf16x8, ld16(row + grp * 16 + u * 64));
  }
}

template <bool F8>
__device__ __forceinline__ IxkFrag<F8> ixk_zero() {
  if constexpr (F8) return 0l;
  else return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
}

// Q^T fragments of the NCT 16-column tiles of KV head kvh's query heads
// (column = head slot; heads past the group read as zero).  The loads are
// unconditional (from a clamped head) so they go out together with the
// caller's other loads; the zeroing waits for them.
template <int D, int NCT, bool F8>
__device__ __forceinline__ void ixk_q(const IxkParams& p, int b, int kvh, int col, int grp,
                                      IxkFrag<F8> (&qb)[NCT][D / 32]) {
  constexpr int EB = F8 ? 1 : 2;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int hh = min(ct * 16 + col, p.group - 1);
    ixk_row_frags<D, F8>(p.q + ((size_t)b * p.num_q_heads + kvh * p.group + hh) * D * EB, grp, qb[ct]);
  }
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int u = 0; u < D / 32; ++u)
      if (ct * 16 + col >= p.group) qb[ct][u] = ixk_zero<F8>();
}

// Byte address of key j of (sequence b, KV head kvh), its page read from the
// block table.
template <bool F8>
__device__ __forceinline__ const uint8_t* ixk_key(const IxkParams& p, int b, int kvh, int j, int D) {
  const int P = 1 << p.page_log2;
  const int pg = p.block_table[(size_t)b * p.max_pages + (j >> p.page_log2)];
  return p.k_pages + (((size_t)pg * p.num_kv_heads + kvh) * P + (j & (P - 1))) * (size_t)D * (F8 ? 1 : 2);
}

// K fragments of the 16-key tile at keys key0 .. key0 + 15 (each clamped to
// L - 1): lane (col, grp) holds its channels of key key0 + col.
template <int D, bool F8>
__device__ __forceinline__ void ixk_tile(const IxkParams& p, int b, int kvh, int key0, int L, int col, int grp,
                                         IxkFrag<F8> (&kf)[D / 32]) {
  ixk_row_frags<D, F8>(ixk_key<F8>(p, b, kvh, min(key0 + col, L - 1), D), grp, kf);
}

// Scores of the sampled positions (every 16th) for every head of a KV head,
// into the compact rows samp[b * H_q + h][i] = s_{16 i}; also each row's
// length.  Grid (ceil(max_len / (256 * 4 kIxkSampTiles)), H_kv, B), 256
// threads; a wave scores kIxkSampTiles tiles of 16 sampled positions.
template <int D, int NCT, bool F8>
__global__ __launch_bounds__(256) void ixk_samples(IxkParams p) {
  constexpr int NU = D / 32;
  const int b = blockIdx.z, kvh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int col = lane & 15, grp = lane >> 4;
  const int L = p.seq_lens[b];
  if (blockIdx.x == 0)
    for (int i = tid; i < p.group; i += 256) p.row_len[(size_t)b * p.num_q_heads + kvh * p.group + i] = L;
  const int tile0 = (blockIdx.x * 4 + wave) * kIxkSampTiles;
  if (tile0 * 256 >= L) return;
  IxkFrag<F8> qb[NCT][NU];
  ixk_q<D, NCT, F8>(p, b, kvh, col, grp, qb);
  IxkFrag<F8> kf[kIxkSampTiles][NU];
#pragma unroll
  for (int t = 0; t < kIxkSampTiles; ++t)   // lane col loads sampled position 16 (16 tile + col)
    ixk_row_frags<D, F8>(ixk_key<F8>(p, b, kvh, min((tile0 + t) * 256 + 16 * col, L - 1), D), grp, kf[t]);
#pragma unroll
  for (int t = 0; t < kIxkSampTiles; ++t) {
    const int line = tile0 + t;   // entries 16 line .. + 15
    if (line * 256 >= L) break;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < NU; ++u) acc = ixk_mfma<F8>(kf[t][u], qb[ct][u], acc);
      const int hh = ct * 16 + col;
      if (hh < p.group) {
        float* dst = p.samp + ((size_t)b * p.num_q_heads + kvh * p.group + hh) * p.samp_stride + line * 16 + grp * 4;
        *reinterpret_cast<float4*>(dst) =
            make_float4(acc[0] * p.scale, acc[1] * p.scale, acc[2] * p.scale, acc[3] * p.scale);
      }
    }
  }
}

// The indexer pass fused with the compaction: grid (ceil(max_len /
// kIxkChunk), H_kv, B), 256 threads.  Wave w scores positions
// start + kIxkSeg w .. + kIxkSeg - 1 (segment 4 * chunk + w of every row of
// the KV head) tile by tile and appends, for each head, the positions whose key is
// at least the row's tau_lo, with their keys, in position order: the four
// lanes holding a head's 16 keys of a tile take their slots from ballots
// of the tile's four key columns (no cross-lane exchange).  A head's first
// kIxkStage entries of the segment are staged in LDS and written out at the
// end as whole 16-byte pairs, so the few, scattered entries of a tile do not
// each become a store of their own; entries past them go out directly.  Rows that keep everything
// (k >= L_b) store nothing.
template <int D, int NCT, bool F8>
__global__ __launch_bounds__(256) void ixk_compact(IxkParams p) {
  constexpr int NU = D / 32;
  constexpr int QB = KVSEL_IXK_QB > 0 ? KVSEL_IXK_QB : (D == 128 ? 4 : 8) < kIxkSeg / 16 ? (D == 128 ? 4 : 8) : kIxkSeg / 16;
  __shared__ int page_lds[kIxkChunk / 16 + 2];
  __shared__ uint4 stage[4][16 * NCT][kIxkStage / 2];    // per wave and head slot: entry pairs
  __shared__ int stage_n[4][16 * NCT];
  const int b = blockIdx.z, kvh = blockIdx.y, chunk = blockIdx.x;
  const int L = p.seq_lens[b];
  const int start = chunk * kIxkChunk;
  if (start >= L) return;
  const int n_keys = min(kIxkChunk, L - start);
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int col = lane & 15, grp = lane >> 4;
  const int P = 1 << p.page_log2;
  const int first_page = start >> p.page_log2;
  const int n_pages = ((start + n_keys - 1) >> p.page_log2) - first_page + 1;
  // the page ids, the queries and the rows' bounds are loaded together
  // (one round trip) before the page ids go to LDS
  static_assert(kIxkChunk / 16 + 2 <= 256, "one page id per thread");
  const int pg_id = tid < n_pages ? p.block_table[(size_t)b * p.max_pages + first_page + tid] : 0;
  IxkFrag<F8> qb[NCT][NU];
  const bool keep_all = p.topk >= L;
  uint32_t tau[NCT];
  size_t rowi[NCT];
  bool on[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    rowi[ct] = (size_t)b * p.num_q_heads + kvh * p.group + min(ct * 16 + col, p.group - 1);
    tau[ct] = p.tau[rowi[ct]];   // read for every lane; used only where `on`
  }
  ixk_q<D, NCT, F8>(p, b, kvh, col, grp, qb);
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    on[ct] = ct * 16 + col < p.group && !keep_all;
    if (!on[ct]) tau[ct] = 0xFFFFFFFFu;
  }
  if (tid < n_pages) page_lds[tid] = pg_id;
  __syncthreads();
  const int wbase = wave * kIxkSeg;
  if (wbase >= n_keys) return;
  const int seg = chunk * 4 + wave;
  const size_t head_stride = (size_t)P * D * (F8 ? 1 : 2);
  const size_t page_stride = head_stride * p.num_kv_heads;
  auto krow = [&](int key) -> const uint8_t* {
    const int j = start + key;
    const int pg = page_lds[(j >> p.page_log2) - first_page];
    return p.k_pages + (size_t)pg * page_stride + kvh * head_stride + (size_t)(j & (P - 1)) * D * (F8 ? 1 : 2);
  };
  constexpr int nt = kIxkSeg / 16;
  static_assert(nt % QB == 0, "whole load batches per segment");
  const uint64_t mine = 0x0001000100010001ull << col;          // lanes col + 16 g
  // The bound as a float: for a score s (never NaN), key(s) >= tau exactly
  // when s >= the float whose key is tau (-0 and +0 share one key and
  // compare equal).  Bounds at or below key(-inf) (tau = 0: store every
  // position) become -inf; bounds above key(+inf), and heads that store
  // nothing, a NaN that no score reaches.
  float tau_f[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const uint32_t t = tau[ct];
    const float x = __uint_as_float((t & 0x80000000u) ? (t & 0x7FFFFFFFu) : ~t);
    tau_f[ct] = !on[ct] ? __builtin_nanf("") : t < 0x00800000u ? -__builtin_inff() : x;
  }
  int base[NCT];
  uint2* slot[NCT];     // this head's entries of the segment
  uint2* st[NCT];       // and their LDS stage
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    base[ct] = 0;
    slot[ct] = p.slots + (rowi[ct] * p.n_oseg + seg) * kIxkSeg;
    st[ct] = reinterpret_cast<uint2*>(stage[wave][ct * 16 + col]);
  }
  // whole segments test no key against the row's end
  const bool whole = wbase + kIxkSeg <= n_keys;
  for (int t0 = 0; t0 < nt; t0 += QB) {
    IxkFrag<F8> kb[QB][NU];
#pragma unroll
    for (int t = 0; t < QB; ++t)   // a lane reads its channels of key col (a tile's rows whole)
      ixk_row_frags<D, F8>(krow(min(wbase + (t0 + t) * 16 + col, n_keys - 1)), grp, kb[t]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < QB; ++t) {
      const int k0 = wbase + (t0 + t) * 16 + grp * 4;   // chunk-relative key of acc[0]
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < NU; ++u) acc = ixk_mfma<F8>(kb[t][u], qb[ct][u], acc);
        float sc[4];
        bool f[4];
        int before = 0, tot = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sc[i] = acc[i] * p.scale;
          f[i] = (whole || k0 + i < n_keys) && sc[i] >= tau_f[ct];
          // the head's four lanes are col, col + 16, col + 32, col + 48: its
          // entries of this tile in lanes below this one, and in all four
          const uint64_t m = __ballot(f[i]) & mine;
          before = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, before));
          tot += __popcll(m);
        }
        if (f[0] | f[1] | f[2] | f[3]) {
          int pos = base[ct] + before;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (f[i]) {
              const uint2 e = make_uint2((uint32_t)(start + k0 + i), order_key(sc[i]));
              if (pos < kIxkStage) st[ct][pos] = e;
              else slot[ct][pos] = e;
              ++pos;
            }
        }
        base[ct] += tot;
      }
    }
  }
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
    if (grp == 0) {
      const int n = on[ct] ? base[ct] : 0;
      stage_n[wave][ct * 16 + col] = n;
      if (ct * 16 + col < p.group) p.counts[rowi[ct] * p.n_oseg + seg] = n;
    }
  // This wave's staged pairs out: head slot hs, pair i; LDS operations of a
  // wave complete in order, and the fences keep the compiler from moving the
  // reads above the writes.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  constexpr int kPairs = kIxkStage / 2;
  for (int x = lane; x < 16 * NCT * kPairs; x += kWave) {
    const int hs = x / kPairs, i = x % kPairs;
    if (hs < p.group && 2 * i < min(stage_n[wave][hs], kIxkStage)) {
      const size_t row = (size_t)b * p.num_q_heads + kvh * p.group + hs;
      reinterpret_cast<uint4*>(p.slots + (row * p.n_oseg + seg) * kIxkSeg)[i] = stage[wave][hs][i];
    }
  }
}

// Scores of row r (positions 0 .. L - 1) into dst, by the whole workgroup
// (kFinThreads threads): the fallback of a row whose stored entries do not
// decide its selection.  Head h sits in its column slot of the indexer's
// tile (the same MFMA element), so the values are those of the other passes.
template <int D, bool F8>
__device__ void ixk_row_scores(const IxkParams& p, int r, float* dst) {
  constexpr int NU = D / 32;
  const int b = r / p.num_q_heads, h = r % p.num_q_heads;
  const int kvh = h / p.group, hs = (h - kvh * p.group) % 16;
  const int L = p.seq_lens[b];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int col = lane & 15, grp = lane >> 4;
  IxkFrag<F8> qb[NU];
  ixk_row_frags<D, F8>(p.q + ((size_t)b * p.num_q_heads + h) * D * (F8 ? 1 : 2), grp, qb);
#pragma unroll
  for (int u = 0; u < NU; ++u)
    if (col != hs) qb[u] = ixk_zero<F8>();
  const int n_tiles = (L + 15) / 16;
  for (int t = wave; t < n_tiles; t += kFinThreads / kWave) {
    IxkFrag<F8> kf[NU];
    ixk_tile<D, F8>(p, b, kvh, t * 16, L, col, grp, kf);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < NU; ++u) acc = ixk_mfma<F8>(kf[u], qb[u], acc);
    if (col == hs) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = t * 16 + grp * 4 + i;
        if (j < L) dst[j] = acc[i] * p.scale;
      }
    }
  }
  __syncthreads();
}

// The final selection of the fused path: segments of kIxkSeg positions; a
// row that falls back first has its scores computed into its own slot area
// (sp.rp.scores and sp.rp.stride point there), which it no longer needs.
template <int D, bool F8>
__global__ __launch_bounds__(kFinThreads) void ixk_final(SplitParams sp, IxkParams ip) {
  __shared__ RowLds sh;
  __shared__ DigitLds L;
  __shared__ int seg_pre[kIxkSegs + 1];
  split_final_row<kIxkSeg, kIxkSegs / kFinThreads>(sp, sh, L, seg_pre, [&](int r) {
    ixk_row_scores<D, F8>(ip, r, const_cast<float*>(sp.rp.scores) + (size_t)r * sp.rp.stride);
  });
}

// Row lengths of the unfused path (row r = b * H_q + h has L_b positions).
__global__ void ixk_row_len(const int32_t* seq_lens, int num_q_heads, int rows, int32_t* row_len) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < rows) row_len[r] = seq_lens[r / num_q_heads];
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
                 reinterpret_cast<uint2*>(ws + o_slots), (max_len + kOutSeg - 1) / kOutSeg, max_len, nullptr, 0};
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

namespace {

inline size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

// The fused path takes the shapes the split selection takes, with rows of at
// most kIxkSegs segments of kIxkSeg positions.
inline bool ixk_fused(int rows, int max_len, int topk) {
  return use_split(rows, max_len, topk) && max_len <= kIxkSegs * kIxkSeg;
}

// Workspace of the fused path: compact samples, row lengths, tau_lo, the
// segment counts and the stored entries (a fallback row's scores reuse its
// own entry area); of the other path: the logits, row lengths and the
// selection's own workspace.
struct IxkLayout {
  size_t o_row_len, o_tau, o_counts, o_slots, total;
  int samp_stride, n_oseg;
  int64_t stride;   // the other path: floats per logits row
};

inline IxkLayout ixk_layout(int num_seqs, int num_q_heads, int max_len, int topk) {
  IxkLayout l{};
  const size_t rows = (size_t)num_seqs * num_q_heads;
  if (ixk_fused((int)rows, max_len, topk)) {
    l.samp_stride = 16 * ((max_len + 255) / 256);
    l.n_oseg = (max_len + kIxkSeg - 1) / kIxkSeg;
    l.o_row_len = al256(rows * l.samp_stride * sizeof(float));
    l.o_tau = l.o_row_len + al256(rows * sizeof(int32_t));
    l.o_counts = l.o_tau + al256(rows * sizeof(uint32_t));
    l.o_slots = l.o_counts + al256(rows * l.n_oseg * sizeof(int));
    l.total = l.o_slots + al256(rows * l.n_oseg * kIxkSeg * sizeof(uint2));
  } else {
    l.stride = ((int64_t)max_len + 3) & ~int64_t(3);
    l.o_row_len = al256(rows * (size_t)l.stride * sizeof(float));
    l.o_slots = l.o_row_len + al256(rows * sizeof(int32_t));   // the selection's workspace
    l.total = l.o_slots + al256(select_workspace_bytes((int)rows, max_len, 0));
  }
  return l;
}

template <int D, int NCT, bool F8>
hipError_t launch_ixk(const IxkParams& ip, const SplitParams& sp, int num_seqs, int max_len, hipStream_t stream) {
  const int rows = num_seqs * ip.num_q_heads;
  const int lines = (max_len + 255) / 256;
  hipLaunchKernelGGL((ixk_samples<D, NCT, F8>), dim3((lines + 4 * kIxkSampTiles - 1) / (4 * kIxkSampTiles),
                     ip.num_kv_heads, num_seqs), dim3(256), 0, stream, ip);
  hipLaunchKernelGGL((select_split_sample<true, true>), dim3(rows), dim3(kSampleThreads), 0, stream, sp);
  hipLaunchKernelGGL((ixk_compact<D, NCT, F8>), dim3((max_len + kIxkChunk - 1) / kIxkChunk, ip.num_kv_heads, num_seqs),
                     dim3(256), 0, stream, ip);
  hipLaunchKernelGGL((ixk_final<D, F8>), dim3(rows), dim3(kFinThreads), 0, stream, sp, ip);
  return hipGetLastError();
}

}  // namespace

size_t indexer_topk_workspace_bytes(int num_seqs, int num_q_heads, int max_seq_len, int topk) {
  return ixk_layout(num_seqs, num_q_heads, max_seq_len, topk).total;
}

hipError_t launch_indexer_topk(const IndexerTopkArgs& a, hipStream_t stream) {
  const IxkLayout l = ixk_layout(a.num_seqs, a.num_q_heads, a.max_seq_len, a.topk);
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  const int rows = a.num_seqs * a.num_q_heads;
  int32_t* row_len = reinterpret_cast<int32_t*>(ws + l.o_row_len);
  if (!ixk_fused(rows, a.max_seq_len, a.topk)) {
    // the logits in the workspace, then the row selection on them
    float* logits = reinterpret_cast<float*>(ws);
    hipLaunchKernelGGL(ixk_row_len, dim3((rows + 255) / 256), dim3(256), 0, stream, a.seq_lens, a.num_q_heads,
                       rows, row_len);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.fp8) {
      e = launch_indexer_fp8(a.k_pages, a.block_table, a.seq_lens, a.q, a.num_seqs, a.num_kv_heads, a.num_q_heads,
                             a.head_dim, a.page_size, a.max_pages, a.max_seq_len, a.scale, logits, l.stride, stream);
      if (e != hipSuccess) return e;
      return launch_select(logits, l.stride, row_len, rows, a.max_seq_len, 0, 0, nullptr, a.topk, 0, 0, a.keep,
                           a.keep_stride, a.counts, ws + l.o_slots, stream);
    }
    const DecodePlan pl = plan_decode(a.num_seqs, a.num_kv_heads, a.num_q_heads, a.head_dim, a.max_seq_len, false);
    DecodeArgs d{};
    d.k_pages = a.k_pages;
    d.block_table = a.block_table;
    d.seq_lens = a.seq_lens;
    d.q = a.q;
    d.num_seqs = a.num_seqs;
    d.num_kv_heads = a.num_kv_heads;
    d.num_q_heads = a.num_q_heads;
    d.head_dim = a.head_dim;
    d.page_size = a.page_size;
    d.max_pages = a.max_pages;
    d.max_seq_len = a.max_seq_len;
    d.bf16 = true;
    d.scale = a.scale;
    d.probs = logits;
    d.probs_stride = l.stride;
    d.emit_logits = true;
    d.decay = 1.f;
    d.workspace = ws;   // the logits-only pass uses no workspace
    e = launch_decode(d, pl, stream);
    if (e != hipSuccess) return e;
    return launch_select(logits, l.stride, row_len, rows, a.max_seq_len, 0, 0, nullptr, a.topk, 0, 0, a.keep,
                         a.keep_stride, a.counts, ws + l.o_slots, stream);
  }
  IxkParams ip{};
  ip.k_pages = static_cast<const uint8_t*>(a.k_pages);
  ip.block_table = a.block_table;
  ip.seq_lens = a.seq_lens;
  ip.q = static_cast<const uint8_t*>(a.q);
  ip.num_kv_heads = a.num_kv_heads;
  ip.num_q_heads = a.num_q_heads;
  ip.group = a.num_q_heads / a.num_kv_heads;
  ip.page_log2 = __builtin_ctz((unsigned)a.page_size);
  ip.max_pages = a.max_pages;
  ip.topk = a.topk;
  ip.scale = a.scale;
  ip.samp = reinterpret_cast<float*>(ws);
  ip.samp_stride = l.samp_stride;
  ip.row_len = row_len;
  ip.tau = reinterpret_cast<uint32_t*>(ws + l.o_tau);
  ip.counts = reinterpret_cast<int*>(ws + l.o_counts);
  ip.slots = reinterpret_cast<uint2*>(ws + l.o_slots);
  ip.n_oseg = l.n_oseg;
  // The selection reads the row lengths the sample pass writes; a fallback
  // row's scores go to its own entry area (n_oseg * kIxkSeg * 2 floats).
  RowsParams rp{reinterpret_cast<const float*>(ws + l.o_slots), (int64_t)l.n_oseg * kIxkSeg * 2, row_len, nullptr,
                a.topk, 0, 0, a.keep, a.keep_stride, a.counts};
  SplitParams sp{rp, reinterpret_cast<uint32_t*>(ws + l.o_tau), reinterpret_cast<int*>(ws + l.o_counts),
                 reinterpret_cast<uint2*>(ws + l.o_slots), l.n_oseg, a.max_seq_len, ip.samp, l.samp_stride};
  const bool two = ip.group > 16;
  auto go = [&](auto f8) {
    constexpr bool F8 = decltype(f8)::value;
    if (a.head_dim == 128)
      return two ? launch_ixk<128, 2, F8>(ip, sp, a.num_seqs, a.max_seq_len, stream)
                 : launch_ixk<128, 1, F8>(ip, sp, a.num_seqs, a.max_seq_len, stream);
    return two ? launch_ixk<64, 2, F8>(ip, sp, a.num_seqs, a.max_seq_len, stream)
               : launch_ixk<64, 1, F8>(ip, sp, a.num_seqs, a.max_seq_len, stream);
  };
  return a.fp8 ? go(std::true_type{}) : go(std::false_type{});
}

bool select_rows_split(int rows, int max_len, int max_budget) { return use_split(rows, max_len, max_budget); }

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
