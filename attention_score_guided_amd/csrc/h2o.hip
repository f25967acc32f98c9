// H2O decode step with per-step eviction.
//
// What is computed ([EVICT] "KV-cache eviction strategies", §4.2 H2O, read
// with the eviction inside the decode loop): the cache of each (sequence,
// KV head) holds a list of kept positions (its slots, ascending) with their
// cumulative scores.  One step
//   1. appends the new token's position L_b - 1 to every list (score 0);
//   2. runs attention of every query head over its KV head's list only, and
//      the exact probability of every listed key;
//   3. folds the group's probabilities into the slot scores,
//      cum = decay * cum + sum over the group of p;
//   4. keeps the first `sinks` slots, the last `window` slots and the top
//      (budget - forced) of the others by score (ties to the lower position),
//      and drops the rest for good: the list shrinks back to the budget.
//
// Kernels: h2o_append_kernel (one thread per list); the split-K sparse
// attention over the lists shared by each group (logits left raw, lse per
// head); h2o_fold_evict_kernel (one workgroup per list: normalise + fold with
// one writer per slot, exact and deterministic, then the common case of a
// decode step, exactly one slot to drop, by an argmin over the middle and a
// shift of the slots after it, all from registers); lists that must shed
// more than one slot (a first step after seeding, a lowered budget) or that
// are longer than the registers hold go through the row selection kernels
// and h2o_compact_kernel (the kept slots moved down in place through LDS).
#include "device_common.hpp"
#include "kvsel_internal.hpp"

#include <algorithm>

namespace kvsel {

namespace {

constexpr int kFoldThreads = 1024;
constexpr int kFoldSlots = 8;         // slots per thread held in registers by the fused kernel (more spills)
constexpr int kCompactThreads = 1024;
constexpr int kCompactChunk = 8192;   // slots staged in LDS per round

__global__ __launch_bounds__(64) void h2o_append_kernel(const int32_t* seq_lens, int num_kv_heads, int rows,
                                                        int32_t* slots, float* slot_cum, int32_t* slot_count,
                                                        int64_t slot_stride) {
  const int r = blockIdx.x * 64 + threadIdx.x;
  if (r >= rows) return;
  const int c = slot_count[r];
  if (c >= slot_stride) return;   // precondition violated: the list is full (left as is)
  slots[(size_t)r * slot_stride + c] = seq_lens[r / num_kv_heads] - 1;
  slot_cum[(size_t)r * slot_stride + c] = 0.f;
  slot_count[r] = c + 1;
}

struct FoldParams {
  int32_t* slots;
  int32_t* slot_count;
  float* slot_cum;
  int64_t slot_stride;
  float* probs;          // [B][H_q][slot_stride] raw logits in, probabilities out
  const float* lse;      // [B][H_q]
  const int32_t* budgets;
  int32_t* gen_len;      // [rows] out: n when the list needs the general selection, else 0
  int num_kv_heads, group, sinks, window, budget;
  bool write_probs;      // the caller asked for the probabilities
  float decay;
};

// Order of the eviction candidates: the lower score goes first, and among
// equal scores the higher slot (the later position) goes first.
__device__ __forceinline__ bool evict_before(float sa, int ia, float sb, int ib) {
  return sa < sb || (sa == sb && ia > ib);
}

// One workgroup per (sequence, KV head) list.
__global__ __launch_bounds__(kFoldThreads) void h2o_fold_evict_kernel(FoldParams p) {
  __shared__ float red_s[kFoldThreads / kWave];
  __shared__ int red_i[kFoldThreads / kWave];
  const size_t row = blockIdx.x;
  const int b = (int)(row / p.num_kv_heads), kvh = (int)(row % p.num_kv_heads);
  const int n = p.slot_count[row];
  const int tid = threadIdx.x;
  const size_t hq0 = (size_t)b * p.num_kv_heads * p.group + (size_t)kvh * p.group;
  int32_t* sl = p.slots + row * p.slot_stride;
  float* cm = p.slot_cum + row * p.slot_stride;
  const bool in_regs = n <= kFoldSlots * kFoldThreads;
  float sc[kFoldSlots];
  int pos[kFoldSlots];
  // ---- fold: p = exp(s - lse) per head of the group, cum = decay cum + sum p
  // The first kFoldSlots slots of each thread stay in registers.  Loads are
  // issued a whole batch at a time (one head of the group per round), so the
  // stores of one round never hold back the loads of the same round.
  float acc[kFoldSlots];
#pragma unroll
  for (int j = 0; j < kFoldSlots; ++j) {
    const int i = tid + j * kFoldThreads;
    acc[j] = 0.f;
    sc[j] = i < n ? cm[i] : 0.f;
    pos[j] = i < n ? sl[i] : 0;
  }
  for (int g = 0; g < p.group; ++g) {
    float* pr = p.probs + (hq0 + g) * p.slot_stride;
    const float l = p.lse[hq0 + g];
    float v[kFoldSlots];
#pragma unroll
    for (int j = 0; j < kFoldSlots; ++j) {
      const int i = tid + j * kFoldThreads;
      v[j] = i < n ? pr[i] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kFoldSlots; ++j) {
      const int i = tid + j * kFoldThreads;
      v[j] = (l == kNegInf || i >= n) ? 0.f : exp2_hw((v[j] - l) * kLog2e);
      acc[j] += v[j];
    }
    if (p.write_probs) {
#pragma unroll
      for (int j = 0; j < kFoldSlots; ++j) {
        const int i = tid + j * kFoldThreads;
        if (i < n) pr[i] = v[j];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kFoldSlots; ++j) {
    const int i = tid + j * kFoldThreads;
    sc[j] = fmaf(p.decay, sc[j], acc[j]);
    if (i < n) cm[i] = sc[j];
  }
  // lists too long for the registers: slot by slot
  for (int i = tid + kFoldSlots * kFoldThreads; i < n; i += kFoldThreads) {
    float a = 0.f;
    for (int g = 0; g < p.group; ++g) {
      float* pr = p.probs + (hq0 + g) * p.slot_stride + i;
      const float l = p.lse[hq0 + g];
      const float v = l == kNegInf ? 0.f : exp2_hw((*pr - l) * kLog2e);
      if (p.write_probs) *pr = v;
      a += v;
    }
    cm[i] = fmaf(p.decay, cm[i], a);
  }
  // ---- eviction --------------------------------------------------------------
  const int B = p.budgets ? p.budgets[row] : p.budget;
  const int lo = min(p.sinks, n), hi = max(n - p.window, 0);
  int gen = 0;
  if (n > B && hi > lo) {
    const int k = max(0, B - (lo + (n - hi)));
    if (hi - lo - k != 1 || !in_regs) {
      gen = n;   // more than one slot to drop: the general selection
    } else {
      // exactly one: the first in eviction order among slots [lo, hi)
      float bs = __builtin_inff();
      int bi = -1;
#pragma unroll
      for (int j = 0; j < kFoldSlots; ++j) {
        const int i = tid + j * kFoldThreads;
        if (i >= lo && i < hi && (bi < 0 || evict_before(sc[j], i, bs, bi))) { bs = sc[j]; bi = i; }
      }
      for (int off = kWave / 2; off > 0; off /= 2) {
        const float os = __shfl_xor(bs, off, kWave);
        const int oi = __shfl_xor(bi, off, kWave);
        if (oi >= 0 && (bi < 0 || evict_before(os, oi, bs, bi))) { bs = os; bi = oi; }
      }
      if (tid % kWave == 0) { red_s[tid / kWave] = bs; red_i[tid / kWave] = bi; }
      __syncthreads();
      bs = red_s[0];
      bi = red_i[0];
      for (int w = 1; w < kFoldThreads / kWave; ++w)
        if (red_i[w] >= 0 && (bi < 0 || evict_before(red_s[w], red_i[w], bs, bi))) { bs = red_s[w]; bi = red_i[w]; }
      // every slot after the evicted one moves down by one, from registers
#pragma unroll
      for (int j = 0; j < kFoldSlots; ++j) {
        const int i = tid + j * kFoldThreads;
        if (i > bi && i < n) { sl[i - 1] = pos[j]; cm[i - 1] = sc[j]; }
      }
      if (tid == 0) p.slot_count[row] = n - 1;
    }
  }
  if (tid == 0) p.gen_len[row] = gen;
}

struct CompactParams {
  int32_t* slots;
  float* slot_cum;
  int32_t* slot_count;
  int64_t slot_stride;
  const int32_t* sel;       // [rows][sel_stride] kept slot numbers, ascending
  const int32_t* sel_count; // [rows]
  const int32_t* gen_len;   // [rows] 0: the list was settled by the fused kernel
  int sel_stride;
};

// The kept slots (ascending slot numbers sel[i] >= i) move down to 0..m-1.
// Chunk by chunk: every read of a chunk names a slot >= its first index,
// which no earlier chunk has written, so staging one chunk in LDS suffices.
__global__ __launch_bounds__(kCompactThreads) void h2o_compact_kernel(CompactParams p) {
  __shared__ int32_t pos_lds[kCompactChunk];
  __shared__ float cum_lds[kCompactChunk];
  const size_t row = blockIdx.x;
  if (p.gen_len[row] == 0) return;   // settled by the fused kernel
  const int n = p.slot_count[row];
  const int m = p.sel_count[row];
  if (m == n) return;   // every slot kept: the list is unchanged
  int32_t* sl = p.slots + row * p.slot_stride;
  float* cm = p.slot_cum + row * p.slot_stride;
  const int32_t* sel = p.sel + row * p.sel_stride;
  for (int i0 = 0; i0 < m; i0 += kCompactChunk) {
    const int len = min(kCompactChunk, m - i0);
    for (int i = threadIdx.x; i < len; i += kCompactThreads) {
      const int s = sel[i0 + i];
      pos_lds[i] = sl[s];
      cum_lds[i] = cm[s];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < len; i += kCompactThreads) {
      sl[i0 + i] = pos_lds[i];
      cm[i0 + i] = cum_lds[i];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) p.slot_count[row] = m;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace layout: [sparse partials] [lse B*Hq] [logits B*Hq*slot_stride
// when the caller passes no probs] [sel rows*sel_stride] [sel_count rows]
// [gen_len rows] [row selection workspace].
struct H2oLayout {
  size_t sparse, lse, logits, sel, sel_count, gen_len, select, total;
  int sel_stride;
};

H2oLayout h2o_layout(int num_seqs, int num_kv_heads, int num_q_heads, int head_dim, int64_t slot_stride,
                     int sinks, int window, int budget) {
  H2oLayout l{};
  const size_t rows = (size_t)num_seqs * num_kv_heads;
  const size_t bh = (size_t)num_seqs * num_q_heads;
  l.sel_stride = (int)std::max<long long>(1, std::min<long long>(slot_stride, std::max<long long>(budget, (long long)sinks + window)));
  l.sparse = align256(sparse_workspace_bytes(num_seqs, num_q_heads, head_dim, (int)slot_stride));
  l.lse = align256(bh * sizeof(float));
  l.logits = align256(bh * (size_t)slot_stride * sizeof(float));
  l.sel = align256(rows * (size_t)l.sel_stride * sizeof(int32_t));
  l.sel_count = align256(rows * sizeof(int32_t));
  l.gen_len = align256(rows * sizeof(int32_t));
  l.select = select_workspace_bytes((int)rows, (int)slot_stride, 0);
  l.total = l.sparse + l.lse + l.logits + l.sel + l.sel_count + l.gen_len + l.select;
  return l;
}

}  // namespace

size_t h2o_workspace_bytes(int num_seqs, int num_kv_heads, int num_q_heads, int head_dim, int64_t slot_stride,
                           int sinks, int window, int budget) {
  return h2o_layout(num_seqs, num_kv_heads, num_q_heads, head_dim, slot_stride, sinks, window, budget).total;
}

hipError_t launch_h2o_step(const H2oArgs& a, hipStream_t stream) {
  const SparseArgs& s0 = a.sp;
  const H2oLayout l = h2o_layout(s0.num_seqs, s0.num_kv_heads, s0.num_q_heads, s0.head_dim, a.slot_stride,
                                 a.sinks, a.window, a.budget);
  uint8_t* ws = static_cast<uint8_t*>(s0.workspace);
  uint8_t* w_sparse = ws;
  float* lse = reinterpret_cast<float*>(ws + l.sparse);
  float* logits = reinterpret_cast<float*>(ws + l.sparse + l.lse);
  int32_t* sel = reinterpret_cast<int32_t*>(ws + l.sparse + l.lse + l.logits);
  int32_t* sel_count = reinterpret_cast<int32_t*>(ws + l.sparse + l.lse + l.logits + l.sel);
  int32_t* gen_len = reinterpret_cast<int32_t*>(ws + l.sparse + l.lse + l.logits + l.sel + l.sel_count);
  uint8_t* w_select = ws + l.sparse + l.lse + l.logits + l.sel + l.sel_count + l.gen_len;
  const int rows = s0.num_seqs * s0.num_kv_heads;

  hipLaunchKernelGGL(h2o_append_kernel, dim3((rows + 63) / 64), dim3(64), 0, stream, s0.seq_lens,
                     s0.num_kv_heads, rows, a.slots, a.slot_cum, a.slot_count, a.slot_stride);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  SparseArgs sp = s0;
  sp.indices = a.slots;
  sp.idx_stride = a.slot_stride;
  sp.counts = a.slot_count;
  sp.idx_heads = s0.num_kv_heads;
  sp.max_count = (int)a.slot_stride;
  sp.probs = s0.probs ? s0.probs : logits;
  sp.raw_logits = true;
  sp.lse_out = lse;
  sp.workspace = w_sparse;
  e = launch_sparse(sp, stream);
  if (e != hipSuccess) return e;

  FoldParams fp{a.slots, a.slot_count, a.slot_cum, a.slot_stride, sp.probs, lse, a.budgets, gen_len,
                s0.num_kv_heads, s0.num_q_heads / s0.num_kv_heads, a.sinks, a.window, a.budget,
                s0.probs != nullptr, a.decay};
  hipLaunchKernelGGL(h2o_fold_evict_kernel, dim3((unsigned)rows), dim3(kFoldThreads), 0, stream, fp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  // General selection for the lists flagged above (the others have length 0
  // here, which the selection settles at once).
  e = launch_select(a.slot_cum, a.slot_stride, gen_len, rows, (int)a.slot_stride, a.sinks, a.window, a.budgets,
                    a.budget, 0, 0, sel, l.sel_stride, sel_count, w_select, stream);
  if (e != hipSuccess) return e;

  CompactParams cp{a.slots, a.slot_cum, a.slot_count, a.slot_stride, sel, sel_count, gen_len, l.sel_stride};
  hipLaunchKernelGGL(h2o_compact_kernel, dim3((unsigned)rows), dim3(kCompactThreads), 0, stream, cp);
  return hipGetLastError();
}

}  // namespace kvsel
