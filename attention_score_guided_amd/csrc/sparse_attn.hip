// Sparse attention over an index set ([LONGCTX] "Long context, KV eviction
// and sparse attention", sparse-attention experiment: logits outside the
// selection are masked before the softmax, i.e. the softmax runs over the
// selected keys only; a DeepSeek-style indexer picks 2048 keys per query).
//
// Split-K over the index list: one workgroup takes a slice of up to kSlice
// listed positions of one (sequence, set) and the gt query heads that read the
// set (gt = 1 for per-query-head sets, the group for sets shared by a KV
// head).  Each listed position is gathered through the block table: 16-byte
// lane segments of the key row, dot products reduced across the row's lanes
// with DPP, logits in LDS; chunk max / sum of exp; P.V over the gathered
// value rows.  The partials (m, l, o) are combined per query head into out
// and lse; listed probabilities are normalised in place when requested.
// Entries < 0 and slots past the set's count are ignored.
#include "device_common.hpp"
#include "kvsel_internal.hpp"

namespace kvsel {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
#ifndef KVSEL_SPARSE_SLICE
#define KVSEL_SPARSE_SLICE 128   // 256 measured 15% slower on 2048-entry per-head sets, 3% on 5000-entry shared lists
#endif
#ifndef KVSEL_SPARSE_UNROLL
#define KVSEL_SPARSE_UNROLL 8
#endif
constexpr int kSlice = KVSEL_SPARSE_SLICE;    // listed positions per workgroup
constexpr int kUnroll = KVSEL_SPARSE_UNROLL;  // gathered rows in flight per lane

struct SparseParams {
  const uint8_t* k_pages;
  const uint8_t* v_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint8_t* q;
  const int32_t* indices;   // [B][idx_heads][idx_stride]
  int64_t idx_stride;
  const int32_t* counts;    // [B][idx_heads], read clamped to max_count
  int num_kv_heads, num_q_heads, idx_heads, page_log2, max_pages, n_chunks, max_count;
  bool append_current;      // entry `count` (< max_count) is position seq_lens[b] - 1
  float scale;
  float* probs;             // [B][Hq][idx_stride] raw logits written here, or null
  float* part_o;            // [B][Hq][n_chunks][D]
  float2* part_ml;          // [B][Hq][n_chunks]
};

template <bool BF16, int D, int GT>
__global__ __launch_bounds__(kThreads) void sparse_partial(SparseParams p) {
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int EPL = 16 / EB;
  constexpr int LPK = D / EPL;
  constexpr int KPW = kWave / LPK;
  constexpr int KPI = kWaves * KPW;
  static_assert(LPK >= GT, "a key row must span at least one lane per head");

  __shared__ float s_lds[GT][kSlice];
  __shared__ float red[kWaves][GT][D];
  __shared__ float2 ml_lds[GT];
  __shared__ long long off_lds[kSlice];     // byte offset of the listed row in a head's pages, or -1

  const int chunk = blockIdx.x;
  const int set = blockIdx.y;                 // 0 .. idx_heads-1
  const int b = blockIdx.z;
  const int G = p.num_q_heads / p.num_kv_heads;
  const bool shared = p.idx_heads != p.num_q_heads;
  const int h0 = shared ? set * G : set;      // first query head served
  const int kvh = h0 / G;
  // A count above max_count is a caller error; clamping it keeps every
  // access inside the index rows and the workspace the grid was sized for.
  const int listed = min(p.counts[(size_t)b * p.idx_heads + set], p.max_count);
  const bool app = p.append_current && listed < p.max_count;
  const int count = listed + (app ? 1 : 0);
  const int start = chunk * kSlice;
  if (start >= count) return;
  const int n = min(kSlice, count - start);
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int seg = lane % LPK, slot = lane / LPK;
  const int P = 1 << p.page_log2;
  const int* list = p.indices + ((size_t)b * p.idx_heads + set) * p.idx_stride + start;
  const int L = p.seq_lens[b];
  const size_t head_stride = (size_t)P * D * EB;
  const size_t page_stride = head_stride * p.num_kv_heads;
  // Row offsets of the listed positions, resolved through the block table
  // once, so the gathers below need no dependent load.
  for (int i = tid; i < kSlice; i += kThreads) {
    const int j = i >= n ? -1 : start + i == listed ? L - 1 : list[i];
    long long off = -1;
    if (j >= 0 && j < L) {
      const int pg = p.block_table[(size_t)b * p.max_pages + (j >> p.page_log2)];
      off = (long long)((size_t)pg * page_stride + kvh * head_stride + (size_t)(j & (P - 1)) * D * EB);
    }
    off_lds[i] = off;
  }
  uint32_t qw[GT][4];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    const uint4 v = ld16(p.q + (((size_t)b * p.num_q_heads + h0 + h) * D + seg * EPL) * EB);
    qw[h][0] = v.x; qw[h][1] = v.y; qw[h][2] = v.z; qw[h][3] = v.w;
  }
  __syncthreads();

  // Lane segment of listed row i (null when the entry is ignored).
  auto row_seg = [&](const uint8_t* base, int i) -> const uint8_t* {
    const long long off = i < n ? off_lds[i] : -1;
    return off >= 0 ? base + off + seg * 16 : nullptr;
  };

  // ---- logits of the listed positions -------------------------------------
  // kUnroll rows per lane are loaded before any is used.
  for (int i0 = 0; i0 < n; i0 += KPI * kUnroll) {
    uint4 kr[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint8_t* rp = row_seg(p.k_pages, i0 + u * KPI + wave * KPW + slot);
      kr[u] = rp ? ld16(rp) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = i0 + u * KPI + wave * KPW + slot;
      float part[GT];
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        if constexpr (BF16) {
          float a = dot2_bf16(qw[h][0], kr[u].x, 0.f);
          a = dot2_bf16(qw[h][1], kr[u].y, a);
          a = dot2_bf16(qw[h][2], kr[u].z, a);
          part[h] = dot2_bf16(qw[h][3], kr[u].w, a);
        } else {
          float a = __uint_as_float(qw[h][0]) * __uint_as_float(kr[u].x);
          a = fmaf(__uint_as_float(qw[h][1]), __uint_as_float(kr[u].y), a);
          a = fmaf(__uint_as_float(qw[h][2]), __uint_as_float(kr[u].z), a);
          part[h] = fmaf(__uint_as_float(qw[h][3]), __uint_as_float(kr[u].w), a);
        }
      }
#pragma unroll
      for (int h = 0; h < GT; ++h) part[h] = group_sum<LPK>(part[h]);
      if (i < n) {
        const bool valid = off_lds[i] >= 0;
#pragma unroll
        for (int h = 0; h < GT; ++h)
          if (seg == h) s_lds[h][i] = valid ? part[h] * p.scale : kNegInf;
      }
    }
  }
  __syncthreads();

  // ---- chunk max, raw logits out, exp, sum ---------------------------------
  for (int h = wave; h < GT; h += kWaves) {
    float m = kNegInf;
    for (int i = lane; i < n; i += kWave) m = fmaxf(m, s_lds[h][i]);
    m = wave_max(m);
    const float ms = m == kNegInf ? 0.f : m * kLog2e;
    float* lg = p.probs ? p.probs + ((size_t)b * p.num_q_heads + h0 + h) * p.idx_stride + start : nullptr;
    float l = 0.f;
    for (int i = lane; i < n; i += kWave) {
      const float s = s_lds[h][i];
      if (lg) lg[i] = s;
      const float e = exp2_hw(fmaf(s, kLog2e, -ms));
      s_lds[h][i] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) ml_lds[h] = make_float2(m, l);
  }
  __syncthreads();

  // ---- P.V -----------------------------------------------------------------
  float acc[GT][EPL];
#pragma unroll
  for (int h = 0; h < GT; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  for (int i0 = 0; i0 < n; i0 += KPI * kUnroll) {
    uint4 vb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint8_t* rp = row_seg(p.v_pages, i0 + u * KPI + wave * KPW + slot);
      vb[u] = rp ? ld16(rp) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = i0 + u * KPI + wave * KPW + slot;
      if (i >= n || off_lds[i] < 0) continue;
      const uint4 vr = vb[u];
      float v[EPL];
      if constexpr (BF16) {
        v[0] = bf16lo(vr.x); v[1] = bf16hi(vr.x); v[2] = bf16lo(vr.y); v[3] = bf16hi(vr.y);
        v[4] = bf16lo(vr.z); v[5] = bf16hi(vr.z); v[6] = bf16lo(vr.w); v[7] = bf16hi(vr.w);
      } else {
        v[0] = __uint_as_float(vr.x); v[1] = __uint_as_float(vr.y);
        v[2] = __uint_as_float(vr.z); v[3] = __uint_as_float(vr.w);
      }
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        const float pj = s_lds[h][i];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pj, v[e], acc[h][e]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < GT; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float a = acc[h][e];
#pragma unroll
      for (int off = LPK; off < kWave; off *= 2) a += __shfl_xor(a, off, kWave);
      acc[h][e] = a;
    }
  if (slot == 0) {
#pragma unroll
    for (int h = 0; h < GT; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) red[wave][h][seg * EPL + e] = acc[h][e];
  }
  __syncthreads();
  const size_t base = ((size_t)b * p.num_q_heads + h0) * p.n_chunks + chunk;
  for (int idx = tid; idx < GT * D; idx += kThreads) {
    const int h = idx / D, d = idx % D;
    p.part_o[(base + (size_t)h * p.n_chunks) * D + d] =
        (red[0][h][d] + red[1][h][d]) + (red[2][h][d] + red[3][h][d]);
  }
  if (tid < GT) p.part_ml[base + (size_t)tid * p.n_chunks] = ml_lds[tid];
}

// Per (sequence, query head): combine the chunk partials; out = 0 and
// lse = -inf for an empty set.
struct SparseCombineParams {
  const int32_t* counts;
  const float* part_o;
  const float2* part_ml;
  float* out;
  float* lse_ws;
  int num_q_heads, num_kv_heads, idx_heads, n_chunks, D, max_count;
};

__global__ __launch_bounds__(128) void sparse_combine(SparseCombineParams p) {
  extern __shared__ float w_lds[];            // [n_chunks] exp(m_c - M)
  __shared__ float red[2][2];
  const int bh = blockIdx.x;
  const int b = bh / p.num_q_heads, h = bh % p.num_q_heads;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int set = p.idx_heads == p.num_q_heads ? h : h / G;
  // clamped as in the partial pass: nc <= n_chunks, the LDS and the
  // workspace rows this row owns
  const int count = min(p.counts[(size_t)b * p.idx_heads + set], p.max_count);
  const int nc = (count + kSlice - 1) / kSlice;
  const float2* ml = p.part_ml + (size_t)bh * p.n_chunks;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  // chunk maxima and sums are read once, in parallel, and reduced over the
  // two waves; empty chunks (m = -inf) weigh nothing
  float M = kNegInf;
  for (int c = tid; c < nc; c += 128) M = fmaxf(M, ml[c].x);
  M = wave_max(M);
  if (lane == 0) red[0][wave] = M;
  __syncthreads();
  M = fmaxf(red[0][0], red[0][1]);
  const float Ms = M == kNegInf ? 0.f : M * kLog2e;
  float l = 0.f;
  for (int c = tid; c < nc; c += 128) {
    const float2 v = ml[c];
    const float w = v.x == kNegInf ? 0.f : exp2_hw(fmaf(v.x, kLog2e, -Ms));
    w_lds[c] = w;
    l = fmaf(w, v.y, l);
  }
  l = wave_sum(l);
  if (lane == 0) red[1][wave] = l;
  __syncthreads();
  l = red[1][0] + red[1][1];
  const int d = tid;
  if (d < p.D) {
    // independent loads of the chunk rows, eight in flight
    const float* po = p.part_o + (size_t)bh * p.n_chunks * p.D + d;
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int c = 0;
    for (; c + 8 <= nc; c += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) o[u] = fmaf(w_lds[c + u], po[(size_t)(c + u) * p.D], o[u]);
    }
    for (; c < nc; ++c) o[0] = fmaf(w_lds[c], po[(size_t)c * p.D], o[0]);
    const float os = ((o[0] + o[1]) + (o[2] + o[3])) + ((o[4] + o[5]) + (o[6] + o[7]));
    p.out[(size_t)bh * p.D + d] = l > 0.f ? os / l : 0.f;
  }
  if (tid == 0) p.lse_ws[bh] = l > 0.f ? M + log2_hw(l) * kLn2 : kNegInf;
}

// Listed probabilities: raw logit -> exp(s - lse); ignored entries -> 0.
__global__ __launch_bounds__(256) void sparse_normalize(const int32_t* counts, const int32_t* indices,
                                                        int64_t idx_stride, int num_q_heads,
                                                        int num_kv_heads, int idx_heads, int max_count,
                                                        const float* lse_ws, float* probs) {
  const int bh = blockIdx.y;
  const int b = bh / num_q_heads, h = bh % num_q_heads;
  const int G = num_q_heads / num_kv_heads;
  const int set = idx_heads == num_q_heads ? h : h / G;
  const int count = min(counts[(size_t)b * idx_heads + set], max_count);
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  const int j = indices[((size_t)b * idx_heads + set) * idx_stride + i];
  float* pr = probs + (size_t)bh * idx_stride + i;
  const float lse = lse_ws[bh];
  *pr = (j >= 0 && lse != kNegInf) ? exp2_hw((*pr - lse) * kLog2e) : 0.f;
}

template <bool BF16, int D>
hipError_t launch_sparse_d(const SparseParams& sp, int gt, dim3 grid, hipStream_t s) {
  switch (gt) {
    case 1: hipLaunchKernelGGL((sparse_partial<BF16, D, 1>), grid, dim3(kThreads), 0, s, sp); break;
    case 2: hipLaunchKernelGGL((sparse_partial<BF16, D, 2>), grid, dim3(kThreads), 0, s, sp); break;
    case 4: hipLaunchKernelGGL((sparse_partial<BF16, D, 4>), grid, dim3(kThreads), 0, s, sp); break;
    case 8: hipLaunchKernelGGL((sparse_partial<BF16, D, 8>), grid, dim3(kThreads), 0, s, sp); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

size_t sparse_workspace_bytes(int num_seqs, int num_q_heads, int head_dim, int max_count) {
  const int n_chunks = max(1, (max_count + kSlice - 1) / kSlice);
  const size_t bh = (size_t)num_seqs * num_q_heads;
  return align256(bh * n_chunks * head_dim * sizeof(float)) + align256(bh * n_chunks * sizeof(float2)) +
         align256(bh * sizeof(float));
}

SparsePartials sparse_partials(const SparseArgs& a) {
  const int n_chunks = max(1, (a.max_count + kSlice - 1) / kSlice);
  const size_t bh = (size_t)a.num_seqs * a.num_q_heads;
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  SparsePartials r;
  r.part_o = reinterpret_cast<float*>(ws);
  r.part_ml = reinterpret_cast<float2*>(ws + align256(bh * n_chunks * a.head_dim * sizeof(float)));
  r.n_chunks = n_chunks;
  r.slice = kSlice;
  return r;
}

hipError_t launch_sparse(const SparseArgs& a, hipStream_t stream) {
  const SparsePartials pt = sparse_partials(a);
  const int n_chunks = pt.n_chunks;
  const size_t bh = (size_t)a.num_seqs * a.num_q_heads;
  float* part_o = pt.part_o;
  float2* part_ml = pt.part_ml;
  float* lse_ws = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(part_ml) +
                                           align256(bh * n_chunks * sizeof(float2)));
  const int G = a.num_q_heads / a.num_kv_heads;
  const bool shared = a.idx_heads != a.num_q_heads;
  // Shared sets serve the whole group from one gather (G <= 8 here).
  const int gt = shared ? G : 1;
  SparseParams sp{};
  sp.k_pages = static_cast<const uint8_t*>(a.k_pages);
  sp.v_pages = static_cast<const uint8_t*>(a.v_pages);
  sp.block_table = a.block_table;
  sp.seq_lens = a.seq_lens;
  sp.q = static_cast<const uint8_t*>(a.q);
  sp.indices = a.indices;
  sp.idx_stride = a.idx_stride;
  sp.counts = a.counts;
  sp.num_kv_heads = a.num_kv_heads;
  sp.num_q_heads = a.num_q_heads;
  sp.idx_heads = a.idx_heads;
  sp.page_log2 = __builtin_ctz((unsigned)a.page_size);
  sp.max_pages = a.max_pages;
  sp.n_chunks = n_chunks;
  sp.max_count = a.max_count;
  sp.append_current = a.append_current;
  sp.scale = a.scale;
  sp.probs = a.probs;
  sp.part_o = part_o;
  sp.part_ml = part_ml;
  const dim3 grid(n_chunks, a.idx_heads, a.num_seqs);
  hipError_t e;
  if (a.bf16)
    e = a.head_dim == 128 ? launch_sparse_d<true, 128>(sp, gt, grid, stream)
                          : launch_sparse_d<true, 64>(sp, gt, grid, stream);
  else
    e = a.head_dim == 128 ? launch_sparse_d<false, 128>(sp, gt, grid, stream)
                          : launch_sparse_d<false, 64>(sp, gt, grid, stream);
  if (e != hipSuccess || a.partials_only) return e;
  SparseCombineParams cp{a.counts, part_o, part_ml, a.out, a.lse_out ? a.lse_out : lse_ws, a.num_q_heads,
                         a.num_kv_heads, a.idx_heads, n_chunks, a.head_dim, a.max_count};
  hipLaunchKernelGGL(sparse_combine, dim3((unsigned)bh), dim3(128), n_chunks * sizeof(float), stream, cp);
  e = hipGetLastError();
  if (e != hipSuccess || !a.probs || a.raw_logits) return e;
  hipLaunchKernelGGL(sparse_normalize, dim3((a.max_count + 255) / 256, (unsigned)bh), dim3(256), 0,
                     stream, a.counts, a.indices, a.idx_stride, a.num_q_heads, a.num_kv_heads,
                     a.idx_heads, a.max_count, cp.lse_ws, a.probs);
  return hipGetLastError();
}

}  // namespace kvsel
