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
// Kernels: the split-K partial pass of the sparse attention over the lists
// shared by each group (logits left raw), which reads the current token as
// each list's next entry; h2o_tail_kernel, one workgroup per list, which
//   * appends the current token to the list (score 0),
//   * combines the group's split-K partials into each head's lse and output,
//   * normalises and folds with one writer per slot (exact, deterministic),
//   * settles the common case of a decode step, exactly one slot to drop, by
//     an argmin over the middle and a shift of the slots after it, all from
//     registers,
//   * and selects, inside the same workgroup, the kept slots of a list that
//     must shed more than one (a first step after seeding, a lowered budget)
//     or is longer than the registers hold, then moves them down in place
//     through LDS.
// A decode step is thus two launches.
#include "device_common.hpp"
#include "kvsel_internal.hpp"
#include "row_select.hpp"

#include <algorithm>

namespace kvsel {

namespace {

constexpr int kFoldThreads = 1024;
constexpr int kFoldSlots = 8;         // slots per thread held in registers by the fused kernel (more spills)
constexpr int kCompactChunk = 8192;   // slots staged in LDS per round

constexpr int kMaxGroup = 8;          // query heads sharing a list

struct TailParams {
  const int32_t* seq_lens;
  int32_t* slots;
  int32_t* slot_count;
  float* slot_cum;
  int64_t slot_stride;
  float* probs;          // [B][H_q][slot_stride] raw logits in, probabilities out
  float* out;            // [B][H_q][D]
  const float* part_o;   // split-K partials of the sparse pass (sparse_partials)
  const float2* part_ml;
  int n_chunks, slice, head_dim;
  const int32_t* budgets;
  int32_t* gen_len;      // [rows]: a list's length, for the row selection of a list that sheds > 1 slot
  int32_t* sel;          // [rows][sel_stride]: that selection's kept slot numbers, ascending
  int32_t* sel_count;    // [rows]
  int sel_stride;
  int num_kv_heads, group, sinks, window, budget;
  bool write_probs;      // the caller asked for the probabilities
  float decay;
};

// Order of the eviction candidates: the lower score goes first, and among
// equal scores the higher slot (the later position) goes first.
__device__ __forceinline__ bool evict_before(float sa, int ia, float sb, int ib) {
  return sa < sb || (sa == sb && ia > ib);
}

// The LDS of the general eviction: the row selection, then the compaction's
// staging (one after the other).
struct CompactLds {
  int32_t pos[kCompactChunk];
  float cum[kCompactChunk];
};
union TailLds {
  RowLds sel;
  CompactLds cmp;
};

// One workgroup per (sequence, KV head) list.
__global__ __launch_bounds__(kFoldThreads) void h2o_tail_kernel(TailParams p) {
  __shared__ float red_s[kFoldThreads / kWave];
  __shared__ int red_i[kFoldThreads / kWave];
  __shared__ float head_ms[kMaxGroup], head_l[kMaxGroup], head_lse[kMaxGroup];
  __shared__ TailLds u;
  const size_t row = blockIdx.x;
  const int b = (int)(row / p.num_kv_heads), kvh = (int)(row % p.num_kv_heads);
  // the list as the sparse pass read it: its `listed` slots, then the current
  // token (position L_b - 1, score 0) unless the list is full
  const int listed = p.slot_count[row];
  const bool app = listed < p.slot_stride;
  const int n = listed + (app ? 1 : 0);
  const int L = p.seq_lens[b];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const size_t hq0 = (size_t)b * p.num_kv_heads * p.group + (size_t)kvh * p.group;
  int32_t* sl = p.slots + row * p.slot_stride;
  float* cm = p.slot_cum + row * p.slot_stride;
  const bool in_regs = n <= kFoldSlots * kFoldThreads;
  if (app && tid == 0) sl[listed] = L - 1;
  // The first kFoldSlots slots of each thread stay in registers; their loads
  // go out first, so the combine below hides their latency.
  float sc[kFoldSlots];
  int pos[kFoldSlots];
#pragma unroll
  for (int j = 0; j < kFoldSlots; ++j) {
    const int i = tid + j * kFoldThreads;
    sc[j] = i < listed ? cm[i] : 0.f;
    pos[j] = i < listed ? sl[i] : i == listed ? L - 1 : 0;
  }
  // ---- combine: chunk c of the sparse pass covered listed slots
  // [c slice, (c + 1) slice); per head, M = max m_c, l = sum exp(m_c - M) l_c,
  // lse = M + ln l, out = sum exp(m_c - M) o_c / l (empty chunks weigh nothing)
  const int nc = (n + p.slice - 1) / p.slice;
  for (int g = wave; g < p.group; g += kFoldThreads / kWave) {
    const float2* ml = p.part_ml + (hq0 + g) * p.n_chunks;
    float M = kNegInf;
    for (int c = lane; c < nc; c += kWave) M = fmaxf(M, ml[c].x);
    M = wave_max(M);
    const float Ms = M == kNegInf ? 0.f : M * kLog2e;
    float l = 0.f;
    for (int c = lane; c < nc; c += kWave) {
      const float2 v = ml[c];
      const float w = v.x == kNegInf ? 0.f : exp2_hw(fmaf(v.x, kLog2e, -Ms));
      l = fmaf(w, v.y, l);
    }
    l = wave_sum(l);
    if (lane == 0) {
      head_ms[g] = Ms;
      head_l[g] = l;
      head_lse[g] = l > 0.f ? M + log2_hw(l) * kLn2 : kNegInf;
    }
  }
  __syncthreads();
  for (int i = tid; i < p.group * p.head_dim; i += kFoldThreads) {
    const int g = i / p.head_dim, d = i % p.head_dim;
    const float2* ml = p.part_ml + (hq0 + g) * p.n_chunks;
    const float* po = p.part_o + (hq0 + g) * p.n_chunks * p.head_dim + d;
    const float Ms = head_ms[g];
    // independent loads of the chunk rows, eight in flight
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int c = 0;
    for (; c + 8 <= nc; c += 8) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float mc = ml[c + k].x;
        const float w = mc == kNegInf ? 0.f : exp2_hw(fmaf(mc, kLog2e, -Ms));
        o[k] = fmaf(w, po[(size_t)(c + k) * p.head_dim], o[k]);
      }
    }
    for (; c < nc; ++c) {
      const float mc = ml[c].x;
      const float w = mc == kNegInf ? 0.f : exp2_hw(fmaf(mc, kLog2e, -Ms));
      o[0] = fmaf(w, po[(size_t)c * p.head_dim], o[0]);
    }
    const float os = ((o[0] + o[1]) + (o[2] + o[3])) + ((o[4] + o[5]) + (o[6] + o[7]));
    const float l = head_l[g];
    p.out[(hq0 + g) * p.head_dim + d] = l > 0.f ? os / l : 0.f;
  }
  // ---- fold: p = exp(s - lse) per head of the group, cum = decay cum + sum p
  // Loads are issued a whole batch at a time (one head of the group per
  // round), so the stores of one round never hold back the loads of the same
  // round.
  float acc[kFoldSlots];
#pragma unroll
  for (int j = 0; j < kFoldSlots; ++j) acc[j] = 0.f;
  for (int g = 0; g < p.group; ++g) {
    float* pr = p.probs + (hq0 + g) * p.slot_stride;
    const float l = head_lse[g];
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
      const float l = head_lse[g];
      const float v = l == kNegInf ? 0.f : exp2_hw((*pr - l) * kLog2e);
      if (p.write_probs) *pr = v;
      a += v;
    }
    cm[i] = fmaf(p.decay, i == listed ? 0.f : cm[i], a);
  }
  // ---- eviction --------------------------------------------------------------
  const int B = p.budgets ? p.budgets[row] : p.budget;
  const int lo = min(p.sinks, n), hi = max(n - p.window, 0);
  if (!(n > B && hi > lo)) {
    if (tid == 0) p.slot_count[row] = n;
    return;
  }
  const int k = max(0, B - (lo + (n - hi)));
  if (hi - lo - k == 1 && in_regs) {
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
    if (lane == 0) { red_s[wave] = bs; red_i[wave] = bi; }
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
    return;
  }
  // More than one slot to drop (or a list longer than the registers hold):
  // the row selection over the folded scores, in this workgroup.
  if (tid == 0) p.gen_len[row] = n;
  __syncthreads();   // the folded scores and the length are visible to every thread
  const RowsParams rp{p.slot_cum, p.slot_stride, p.gen_len, p.budgets, p.budget, p.sinks, p.window,
                      p.sel, p.sel_stride, p.sel_count};
  if (n <= kSmallRow) select_row_small(rp, (int)row, u.sel, B);
  else select_row<kFoldThreads>(rp, (int)row, u.sel, B);
  __syncthreads();   // the kept slots are written; u.sel is free
  // The kept slots (ascending slot numbers sel[i] >= i) move down to
  // 0..m-1, chunk by chunk: every read of a chunk names a slot >= its first
  // index, which no earlier chunk has written, so staging one chunk in LDS
  // suffices.
  const int m = p.sel_count[row];
  if (m == n) {   // every slot kept: the list is unchanged
    if (tid == 0) p.slot_count[row] = n;
    return;
  }
  const int32_t* sel = p.sel + row * p.sel_stride;
  for (int i0 = 0; i0 < m; i0 += kCompactChunk) {
    const int len = min(kCompactChunk, m - i0);
    for (int i = tid; i < len; i += kFoldThreads) {
      const int s = sel[i0 + i];
      u.cmp.pos[i] = sl[s];
      u.cmp.cum[i] = cm[s];
    }
    __syncthreads();
    for (int i = tid; i < len; i += kFoldThreads) {
      sl[i0 + i] = u.cmp.pos[i];
      cm[i0 + i] = u.cmp.cum[i];
    }
    __syncthreads();
  }
  if (tid == 0) p.slot_count[row] = m;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace layout: [sparse partials] [logits B*Hq*slot_stride when the
// caller passes no probs] [sel rows*sel_stride] [sel_count rows] [gen_len rows].
struct H2oLayout {
  size_t sparse, logits, sel, sel_count, gen_len, total;
  int sel_stride;
};

H2oLayout h2o_layout(int num_seqs, int num_kv_heads, int num_q_heads, int head_dim, int64_t slot_stride,
                     int sinks, int window, int budget) {
  H2oLayout l{};
  const size_t rows = (size_t)num_seqs * num_kv_heads;
  const size_t bh = (size_t)num_seqs * num_q_heads;
  l.sel_stride = (int)std::max<long long>(1, std::min<long long>(slot_stride, std::max<long long>(budget, (long long)sinks + window)));
  l.sparse = align256(sparse_workspace_bytes(num_seqs, num_q_heads, head_dim, (int)slot_stride));
  l.logits = align256(bh * (size_t)slot_stride * sizeof(float));
  l.sel = align256(rows * (size_t)l.sel_stride * sizeof(int32_t));
  l.sel_count = align256(rows * sizeof(int32_t));
  l.gen_len = align256(rows * sizeof(int32_t));
  l.total = l.sparse + l.logits + l.sel + l.sel_count + l.gen_len;
  return l;
}

}  // namespace

size_t h2o_workspace_bytes(int num_seqs, int num_kv_heads, int num_q_heads, int head_dim, int64_t slot_stride,
                           int sinks, int window, int budget) {
  return h2o_layout(num_seqs, num_kv_heads, num_q_heads, head_dim, slot_stride, sinks, window, budget).total;
}

hipError_t launch_h2o_step(const H2oArgs& a, hipStream_t stream) {
  const SparseArgs& s0 = a.sp;
  if (s0.num_q_heads / s0.num_kv_heads > kMaxGroup) return hipErrorInvalidValue;
  const H2oLayout l = h2o_layout(s0.num_seqs, s0.num_kv_heads, s0.num_q_heads, s0.head_dim, a.slot_stride,
                                 a.sinks, a.window, a.budget);
  uint8_t* ws = static_cast<uint8_t*>(s0.workspace);
  uint8_t* w_sparse = ws;
  float* logits = reinterpret_cast<float*>(ws + l.sparse);
  int32_t* sel = reinterpret_cast<int32_t*>(ws + l.sparse + l.logits);
  int32_t* sel_count = reinterpret_cast<int32_t*>(ws + l.sparse + l.logits + l.sel);
  int32_t* gen_len = reinterpret_cast<int32_t*>(ws + l.sparse + l.logits + l.sel + l.sel_count);
  const int rows = s0.num_seqs * s0.num_kv_heads;

  SparseArgs sp = s0;
  sp.indices = a.slots;
  sp.idx_stride = a.slot_stride;
  sp.counts = a.slot_count;
  sp.idx_heads = s0.num_kv_heads;
  sp.max_count = (int)a.slot_stride;
  sp.probs = s0.probs ? s0.probs : logits;
  sp.raw_logits = true;
  sp.lse_out = nullptr;
  sp.partials_only = true;   // combined per list below
  sp.append_current = true;  // the current token is read as each list's next slot
  sp.workspace = w_sparse;
  hipError_t e = launch_sparse(sp, stream);
  if (e != hipSuccess) return e;

  const SparsePartials pt = sparse_partials(sp);
  TailParams tp{s0.seq_lens, a.slots, a.slot_count, a.slot_cum, a.slot_stride, sp.probs, s0.out, pt.part_o, pt.part_ml,
                pt.n_chunks, pt.slice, s0.head_dim, a.budgets, gen_len, sel, sel_count, l.sel_stride,
                s0.num_kv_heads, s0.num_q_heads / s0.num_kv_heads, a.sinks, a.window, a.budget,
                s0.probs != nullptr, a.decay};
  hipLaunchKernelGGL(h2o_tail_kernel, dim3((unsigned)rows), dim3(kFoldThreads), 0, stream, tp);
  return hipGetLastError();
}

}  // namespace kvsel
