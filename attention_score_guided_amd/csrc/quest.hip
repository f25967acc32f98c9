// Quest page-bound selection over a paged KV cache.
//
// What is computed ([LONGCTX] "Long context, KV eviction and sparse
// attention", sparse-attention experiment, the Quest strategy): for every
// whole page of a sequence, each key channel's minimum and maximum over the
// page's keys bound q.k for any key of the page from above:
//     bound(q, page) = sum_d max(q_d * kmin_d, q_d * kmax_d).
// Per query head the `budget_pages` pages with the largest bounds are chosen
// (ties to the lower page), and every key of the trailing partial page is
// kept as well.  The chosen keys are the index set of a sparse attention call.
//
// Kernels:
//   quest_summary_kernel  one wave per (logical page, KV head, sequence):
//                         the page's key rows streamed once, channel min and
//                         max reduced across the wave, written next to the
//                         page's physical id (exact: min/max of stored values
//                         are stored values, so the summary keeps the cache
//                         dtype).  HBM-bound: P*d*E bytes in, 2*d*E out.
//   quest_bounds_kernel   grid (page chunk, KV head x head group, sequence):
//                         a page's summary is read once for the <= 8 query
//                         heads of a group; lanes own 16-byte channel
//                         segments, the bound is summed across the page's
//                         lanes with DPP.  HBM-bound: 2*d*E bytes per
//                         (page, KV head) in, 4*G bytes out.
//   quest_pick_kernel     one workgroup per (sequence, query head) row of
//                         page bounds: the radix top-k of the row selection
//                         (row_select.hpp), then the chosen pages (ascending)
//                         expanded to token positions, followed by the
//                         partial tail page.  Rows long enough for the split
//                         selection take it, then quest_expand_kernel.
#include "device_common.hpp"
#include "kvsel_internal.hpp"
#include "row_select.hpp"

#include <algorithm>

namespace kvsel {

namespace {

constexpr int kQThreads = 256;
constexpr int kQWaves = kQThreads / kWave;
#ifndef KVSEL_QUEST_U
#define KVSEL_QUEST_U 4          // bounds: wave steps whose summary loads are issued together
#endif
#ifndef KVSEL_QUEST_MIN_WGS
#define KVSEL_QUEST_MIN_WGS 1024 // bounds: fewer pages per workgroup until the grid has this many
#endif

// 16 bytes of the cache dtype widened to fp32 (EPL = 8 bf16 or 4 f32).
template <bool BF16>
__device__ __forceinline__ void widen16(const uint4& w, float* f) {
  if constexpr (BF16) {
    f[0] = bf16lo(w.x); f[1] = bf16hi(w.x); f[2] = bf16lo(w.y); f[3] = bf16hi(w.y);
    f[4] = bf16lo(w.z); f[5] = bf16hi(w.z); f[6] = bf16lo(w.w); f[7] = bf16hi(w.w);
  } else {
    f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
  }
}

// Inverse of widen16 for values that are exactly representable (they came
// from the cache): bf16 keeps the upper half of each fp32 word.
template <bool BF16>
__device__ __forceinline__ uint4 narrow16(const float* f) {
  if constexpr (BF16) {
    auto pk = [](float lo, float hi) { return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u); };
    return make_uint4(pk(f[0], f[1]), pk(f[2], f[3]), pk(f[4], f[5]), pk(f[6], f[7]));
  } else {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
}

struct SummaryParams {
  const uint8_t* k_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  uint8_t* summary;   // [num_pages][H_kv][2][D] cache dtype: min row, then max row
  int num_kv_heads, page_log2, max_pages, first_page;
};

// HEAD_MAJOR: blockIdx.x is the KV head, so consecutive workgroups read the
// head slices of the same pages, one contiguous run of the page layout
// (same-box A/B on the whole 128K cache: 231.7 -> 221.7 us); page-major
// grids serve page counts beyond the grid's y limit.
template <bool BF16, int D, bool HEAD_MAJOR>
__global__ __launch_bounds__(kQThreads) void quest_summary_kernel(SummaryParams p) {
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int EPL = 16 / EB;       // channels per lane segment
  constexpr int LPR = D / EPL;       // lanes per key row
  constexpr int RPW = kWave / LPR;   // key rows per wave load
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int lp = p.first_page + (HEAD_MAJOR ? blockIdx.y : blockIdx.x) * kQWaves + wave;  // from first_page
  const int kvh = HEAD_MAJOR ? blockIdx.x : blockIdx.y, b = blockIdx.z;
  const int P = 1 << p.page_log2;
  if ((long long)(lp + 1) * P > p.seq_lens[b]) return;   // whole pages only
  const int pg = p.block_table[(size_t)b * p.max_pages + lp];
  const uint8_t* base = p.k_pages + ((size_t)pg * p.num_kv_heads + kvh) * (size_t)P * D * EB;
  const int seg = lane % LPR, r0 = lane / LPR;
  float mn[EPL], mx[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) { mn[e] = __builtin_inff(); mx[e] = -__builtin_inff(); }
  // P >= 16 is a multiple of RPW (<= 8): every lane sees P / RPW rows.
  for (int r = r0; r < P; r += 4 * RPW) {
    uint4 w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int rr = min(r + u * RPW, P - 1);   // clamped: a repeated row changes no min/max
      w[u] = ld16_stream(base + ((size_t)rr * D + seg * EPL) * EB);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float f[EPL];
      widen16<BF16>(w[u], f);
#pragma unroll
      for (int e = 0; e < EPL; ++e) { mn[e] = fminf(mn[e], f[e]); mx[e] = fmaxf(mx[e], f[e]); }
    }
  }
#pragma unroll
  for (int off = LPR; off < kWave; off *= 2)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      mn[e] = fminf(mn[e], __shfl_xor(mn[e], off, kWave));
      mx[e] = fmaxf(mx[e], __shfl_xor(mx[e], off, kWave));
    }
  if (r0 == 0) {
    uint8_t* dst = p.summary + ((size_t)pg * p.num_kv_heads + kvh) * 2 * D * EB + seg * 16;
    *reinterpret_cast<uint4*>(dst) = narrow16<BF16>(mn);
    *reinterpret_cast<uint4*>(dst + D * EB) = narrow16<BF16>(mx);
  }
}

struct BoundParams {
  const uint8_t* summary;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint8_t* q;        // [B][H_q][D] cache dtype
  float* bounds;           // [B][H_q][bounds_stride]
  int64_t bounds_stride;
  int32_t* row_pages;      // [B][H_q] whole pages per row
  int num_kv_heads, num_q_heads, group, page_log2, max_pages, pages_per_wg;
};

template <bool BF16, int D, int GT>
__global__ __launch_bounds__(kQThreads) void quest_bounds_kernel(BoundParams p) {
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int EPL = 16 / EB;
  constexpr int LPR = D / EPL;       // lanes per page (8..32)
  constexpr int RPW = kWave / LPR;   // pages per wave step
  constexpr int U = KVSEL_QUEST_U;   // wave steps whose loads are issued together
  const int hgroups = p.group / GT;
  const int kvh = blockIdx.y / hgroups, hg = blockIdx.y % hgroups, b = blockIdx.z;
  const int h0 = kvh * p.group + hg * GT;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int seg = lane % LPR, r0 = lane / LPR;
  const int n_full = p.seq_lens[b] >> p.page_log2;
  if (blockIdx.x == 0 && threadIdx.x < GT) p.row_pages[(size_t)b * p.num_q_heads + h0 + threadIdx.x] = n_full;

  float qf[GT][EPL];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    const uint4 w = *reinterpret_cast<const uint4*>(p.q + (((size_t)b * p.num_q_heads + h0 + h) * D + seg * EPL) * EB);
    widen16<BF16>(w, qf[h]);
  }
  const int p_begin = blockIdx.x * p.pages_per_wg;
  const int p_end = min(p_begin + p.pages_per_wg, n_full);
  const int32_t* bt = p.block_table + (size_t)b * p.max_pages;
  const size_t sum_stride = (size_t)p.num_kv_heads * 2 * D * EB;
  const uint8_t* sbase = p.summary + (size_t)kvh * 2 * D * EB + seg * 16;
  float* brow = p.bounds + ((size_t)b * p.num_q_heads + h0) * p.bounds_stride;
  // The physical page ids of the next step are loaded while this step's
  // summaries are in flight, so the loop carries one memory latency per step.
  constexpr int kStep = kQWaves * RPW * U;
  const int lp_first = p_begin + wave * RPW * U + r0;
  int pg_next[U];
#pragma unroll
  for (int u = 0; u < U; ++u) pg_next[u] = lp_first < p_end ? bt[min(lp_first + u * RPW, p_end - 1)] : 0;
  for (int lp0 = lp_first; lp0 < p_end; lp0 += kStep) {
    uint4 mnw[U], mxw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // clamped page ids: the loads stay unconditional
      const uint8_t* s = sbase + (size_t)pg_next[u] * sum_stride;
      mnw[u] = ld16_stream(s);
      mxw[u] = ld16_stream(s + D * EB);
    }
    if (lp0 + kStep < p_end) {
#pragma unroll
      for (int u = 0; u < U; ++u) pg_next[u] = bt[min(lp0 + kStep + u * RPW, p_end - 1)];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float mn[EPL], mx[EPL];
      widen16<BF16>(mnw[u], mn);
      widen16<BF16>(mxw[u], mx);
      float part[GT];
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) s += fmaxf(qf[h][e] * mn[e], qf[h][e] * mx[e]);
        part[h] = group_sum<LPR>(s);
      }
      const int lp = lp0 + u * RPW;
      if (lp < p_end) {
#pragma unroll
        for (int h = 0; h < GT; ++h)
          if (seg == h) brow[(size_t)h * p.bounds_stride + lp] = part[h];
      }
    }
  }
}

struct ExpandParams {
  const int32_t* seq_lens;
  const int32_t* query_pos;  // [B] or null: keep only positions <= query_pos[b]
  const int32_t* page_idx;   // [rows][page_stride] ascending chosen pages
  const int32_t* page_cnt;   // [rows] or null (no whole page anywhere)
  int page_stride;
  int32_t* out_idx;
  int64_t out_stride;
  int32_t* out_count;
  int num_q_heads, page_log2;
};

// Row r's chosen pages (ascending) expanded to token positions, then the
// partial tail page; with query_pos, only positions <= query_pos[b] (every
// thread of the NT-thread workgroup calls it).
template <int NT>
__device__ void expand_row(const ExpandParams& p, int r) {
  const int b = r / p.num_q_heads;
  const int L = p.seq_lens[b];
  const int P = 1 << p.page_log2;
  const int n_full = L >> p.page_log2;
  const int cnt = p.page_cnt ? min(p.page_cnt[r], n_full) : 0;
  const int chosen = cnt * P;
  const int total = chosen + (L - n_full * P);
  const int32_t* pi = p.page_idx + (size_t)r * p.page_stride;
  int32_t* out = p.out_idx + (size_t)r * p.out_stride;
  if (!p.query_pos) {
    for (int i = threadIdx.x; i < total; i += NT)
      out[i] = i < chosen ? (pi[i >> p.page_log2] << p.page_log2) + (i & (P - 1)) : n_full * P + (i - chosen);
    if (threadIdx.x == 0) p.out_count[r] = total;
    return;
  }
  // The causal cut after the choice: the list is ascending, so the positions
  // <= query_pos form a prefix; every thread runs the same number of rounds
  // so that the block-wide count sees each of them.
  const int limit = p.query_pos[b];
  int kept = 0;
  for (int base = 0; base < total; base += NT) {
    const int i = base + threadIdx.x;
    int v = 0;
    if (i < total) v = i < chosen ? (pi[i >> p.page_log2] << p.page_log2) + (i & (P - 1)) : n_full * P + (i - chosen);
    const bool in = i < total && v <= limit;
    if (in) out[i] = v;
    kept += __syncthreads_count(in);
  }
  if (threadIdx.x == 0) p.out_count[r] = kept;
}

__global__ __launch_bounds__(kQThreads) void quest_expand_kernel(ExpandParams p) {
  expand_row<kQThreads>(p, blockIdx.x);
}

// The row's top pages by bound (when some sequence has a whole page), then
// their expansion, in one workgroup: the chosen page ids written by the
// selection are read back after a barrier.
__global__ __launch_bounds__(kRowThreads) void quest_pick_kernel(RowsParams rp, ExpandParams ep) {
  __shared__ RowLds sh;
  const int r = blockIdx.x;
  if (ep.page_cnt) {
    if (rp.lengths[r] <= kSmallRow) select_row_small(rp, r, sh, rp.max_budget);
    else select_row<kRowThreads>(rp, r, sh, rp.max_budget);
    __syncthreads();
  }
  expand_row<kRowThreads>(ep, r);
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

template <bool BF16, int D>
hipError_t launch_bounds_d(const BoundParams& bp, int gt, dim3 grid, hipStream_t s) {
  switch (gt) {
    case 1: hipLaunchKernelGGL((quest_bounds_kernel<BF16, D, 1>), grid, dim3(kQThreads), 0, s, bp); break;
    case 2: hipLaunchKernelGGL((quest_bounds_kernel<BF16, D, 2>), grid, dim3(kQThreads), 0, s, bp); break;
    case 4: hipLaunchKernelGGL((quest_bounds_kernel<BF16, D, 4>), grid, dim3(kQThreads), 0, s, bp); break;
    case 8: hipLaunchKernelGGL((quest_bounds_kernel<BF16, D, 8>), grid, dim3(kQThreads), 0, s, bp); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool HEAD_MAJOR>
void launch_summary(const QuestArgs& a, dim3 grid, hipStream_t stream, const SummaryParams& sp) {
  if (a.bf16) {
    if (a.head_dim == 128)
      hipLaunchKernelGGL((quest_summary_kernel<true, 128, HEAD_MAJOR>), grid, dim3(kQThreads), 0, stream, sp);
    else
      hipLaunchKernelGGL((quest_summary_kernel<true, 64, HEAD_MAJOR>), grid, dim3(kQThreads), 0, stream, sp);
  } else {
    if (a.head_dim == 128)
      hipLaunchKernelGGL((quest_summary_kernel<false, 128, HEAD_MAJOR>), grid, dim3(kQThreads), 0, stream, sp);
    else
      hipLaunchKernelGGL((quest_summary_kernel<false, 64, HEAD_MAJOR>), grid, dim3(kQThreads), 0, stream, sp);
  }
}

}  // namespace

hipError_t launch_quest_summary(const QuestArgs& a, void* summary, int first_page, hipStream_t stream) {
  SummaryParams sp{};
  sp.k_pages = static_cast<const uint8_t*>(a.k_pages);
  sp.block_table = a.block_table;
  sp.seq_lens = a.seq_lens;
  sp.summary = static_cast<uint8_t*>(summary);
  sp.num_kv_heads = a.num_kv_heads;
  sp.page_log2 = __builtin_ctz((unsigned)a.page_size);
  sp.max_pages = a.max_pages;
  sp.first_page = first_page;
  const int max_whole = a.max_seq_len / a.page_size;
  if (max_whole <= first_page) return hipSuccess;   // no whole page from first_page on
  const int n_grp = (max_whole - first_page + kQWaves - 1) / kQWaves;
  if (n_grp <= 65535) {
    const dim3 grid(a.num_kv_heads, n_grp, a.num_seqs);
    launch_summary<true>(a, grid, stream, sp);
  } else {
    const dim3 grid(n_grp, a.num_kv_heads, a.num_seqs);
    launch_summary<false>(a, grid, stream, sp);
  }
  return hipGetLastError();
}

// Workspace: [bounds (when the caller passes none)] [row_pages] [page_idx]
// [page_cnt] [row selection workspace].
size_t quest_workspace_bytes(int num_seqs, int num_q_heads, int page_size, int max_seq_len, int budget_pages) {
  const size_t rows = (size_t)num_seqs * num_q_heads;
  const int max_whole = max_seq_len / page_size;
  const int kp = std::max(1, budget_pages);
  size_t n = align256(rows * std::max(1, max_whole) * sizeof(float)) + align256(rows * sizeof(int32_t)) +
             align256(rows * kp * sizeof(int32_t)) + align256(rows * sizeof(int32_t));
  if (max_whole > 0) n += select_workspace_bytes((int)rows, max_whole, 0);
  return n;
}

hipError_t launch_quest_select(const QuestArgs& a, const void* summary, const void* q, int budget_pages,
                               const int32_t* query_pos, float* bounds, int64_t bounds_stride, int32_t* out_idx,
                               int64_t out_stride, int32_t* out_count, void* workspace, hipStream_t stream) {
  const size_t rows = (size_t)a.num_seqs * a.num_q_heads;
  const int max_whole = a.max_seq_len / a.page_size;
  const int kp = std::max(1, budget_pages);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* ws_bounds = reinterpret_cast<float*>(ws);
  ws += align256(rows * std::max(1, max_whole) * sizeof(float));
  int32_t* row_pages = reinterpret_cast<int32_t*>(ws);
  ws += align256(rows * sizeof(int32_t));
  int32_t* page_idx = reinterpret_cast<int32_t*>(ws);
  ws += align256(rows * kp * sizeof(int32_t));
  int32_t* page_cnt = reinterpret_cast<int32_t*>(ws);
  ws += align256(rows * sizeof(int32_t));
  const int log2p = __builtin_ctz((unsigned)a.page_size);

  if (max_whole > 0) {
    if (!bounds) {
      bounds = ws_bounds;
      bounds_stride = max_whole;
    }
    BoundParams bp{};
    bp.summary = static_cast<const uint8_t*>(summary);
    bp.block_table = a.block_table;
    bp.seq_lens = a.seq_lens;
    bp.q = static_cast<const uint8_t*>(q);
    bp.bounds = bounds;
    bp.bounds_stride = bounds_stride;
    bp.row_pages = row_pages;
    bp.num_kv_heads = a.num_kv_heads;
    bp.num_q_heads = a.num_q_heads;
    bp.group = a.num_q_heads / a.num_kv_heads;
    bp.page_log2 = log2p;
    bp.max_pages = a.max_pages;
    // 256 pages per workgroup, fewer while the grid has under 1024 workgroups
    const int gt = bp.group >= 8 ? 8 : bp.group;
    const long long cols = (long long)a.num_seqs * a.num_kv_heads * (bp.group / gt);
    int ppw = 256;
    while (ppw > 16 && cols * ((max_whole + ppw - 1) / ppw) < KVSEL_QUEST_MIN_WGS) ppw /= 2;
    bp.pages_per_wg = ppw;
    const dim3 grid((max_whole + ppw - 1) / ppw, a.num_kv_heads * (bp.group / gt), a.num_seqs);
    hipError_t e;
    if (a.bf16) e = a.head_dim == 128 ? launch_bounds_d<true, 128>(bp, gt, grid, stream)
                                      : launch_bounds_d<true, 64>(bp, gt, grid, stream);
    else e = a.head_dim == 128 ? launch_bounds_d<false, 128>(bp, gt, grid, stream)
                               : launch_bounds_d<false, 64>(bp, gt, grid, stream);
    if (e != hipSuccess) return e;
  }
  ExpandParams ep{};
  ep.seq_lens = a.seq_lens;
  ep.query_pos = query_pos;
  ep.page_idx = page_idx;
  ep.page_cnt = max_whole > 0 ? page_cnt : nullptr;
  ep.page_stride = kp;
  ep.out_idx = out_idx;
  ep.out_stride = out_stride;
  ep.out_count = out_count;
  ep.num_q_heads = a.num_q_heads;
  ep.page_log2 = log2p;
  // top budget_pages pages of each (sequence, query head) row, ascending,
  // then their positions
  const RowsParams rp{bounds, bounds_stride, row_pages, nullptr, budget_pages, 0, 0, page_idx, kp, page_cnt};
  if (max_whole > 0 && select_rows_split((int)rows, max_whole, budget_pages)) {
    hipError_t e = launch_select(bounds, bounds_stride, row_pages, (int)rows, max_whole, 0, 0, nullptr,
                                 budget_pages, 0, 0, page_idx, kp, page_cnt, ws, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(quest_expand_kernel, dim3((unsigned)rows), dim3(kQThreads), 0, stream, ep);
  } else {
    hipLaunchKernelGGL(quest_pick_kernel, dim3((unsigned)rows), dim3(kRowThreads), 0, stream, rp, ep);
  }
  return hipGetLastError();
}

}  // namespace kvsel
