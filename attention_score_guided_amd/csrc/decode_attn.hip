// Score-emitting split-K GQA decode attention over a paged KV cache, with the
// H2O accumulation fused into the normalisation pass.
//
// What is computed ([OFFLOAD] "Sparse attention x KV-cache offloading", §1.1
// and §1.3; [EVICT] "KV-cache eviction strategies", §4.2 H2O): for each
// sequence b and query head h (KV head c = h / G), logits s_j = scale q.k_j
// over all L_b cached keys, the softmax output, the log-sum-exp, every key's
// exact probability p_j = exp(s_j - lse), and cum[b][c][j] += sum over the
// group of p_j.
//
// Kernels (all HBM-bound; K/V are read exactly once):
//   decode_partial  grid (chunk, kv head x head group, sequence).  One
//                   workgroup streams one chunk of keys of one KV head and
//                   serves the `gt` query heads of its group that read it:
//                   phase 1 QK (bf16 pairs through v_dot2_f32_bf16, the
//                   16 B-per-lane key segments reduced across the lanes of a
//                   key with DPP), logits kept in LDS; phase 2 chunk max, raw
//                   logits streamed out, p = exp(s - m) and l = sum p; phase 3
//                   PV with V read once and the per-head p broadcast from LDS.
//                   Writes the chunk partials (m, l, o).
//   decode_combine  grid (sequence x query head): rescales the chunk partials
//                   to the global max, writes out and lse.
//   decode_finalize grid (key block, kv head, sequence): p = exp(s - lse) for
//                   every head of the group, writes probs and folds the group
//                   sum into cum (one writer per cum element: deterministic).
#include "device_common.hpp"
#include "kvsel_internal.hpp"

namespace kvsel {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = 4;

struct PartialParams {
  const uint8_t* k_pages;
  const uint8_t* v_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint8_t* q;
  float* logits;  // [B][Hq][logits_stride] raw logits, or null
  int64_t logits_stride;
  float* part_o;    // [B][Hq][n_chunks][D]
  float2* part_ml;  // [B][Hq][n_chunks]  (chunk max, chunk sum of exp)
  int num_kv_heads, num_q_heads, group, hgroups, page_log2, max_pages, chunk, n_chunks;
  float scale;
};

// Elements of one 16-byte lane segment.
template <bool BF16>
struct Seg;
template <>
struct Seg<true> {
  static constexpr int kElts = 8;
};
template <>
struct Seg<false> {
  static constexpr int kElts = 4;
};

template <bool BF16, int D, int GT, bool HAS_V, bool WRITE_LOGITS>
__global__ __launch_bounds__(kThreads) void decode_partial(PartialParams p) {
  constexpr int EB = BF16 ? 2 : 4;           // bytes per element
  constexpr int EPL = Seg<BF16>::kElts;      // elements per lane segment
  constexpr int LPK = D / EPL;               // lanes per key row
  constexpr int KPW = kWave / LPK;           // keys per wave per load
  constexpr int KPI = kWaves * KPW;          // keys per workgroup per load
  static_assert(LPK >= GT, "a key row must span at least one lane per head");

  extern __shared__ float smem[];
  const int C = p.chunk;
  float* s_lds = smem;                               // [GT][C]
  float* red = smem + GT * C;                        // [kWaves][GT][D]
  float2* ml_lds = reinterpret_cast<float2*>(red + kWaves * GT * D);  // [GT]
  int* page_lds = reinterpret_cast<int*>(ml_lds + GT);                // [C/16 + 1]

  const int chunk_id = blockIdx.x;
  const int kvh = blockIdx.y / p.hgroups;
  const int hg = blockIdx.y % p.hgroups;
  const int b = blockIdx.z;
  const int L = p.seq_lens[b];
  const int start = chunk_id * C;
  if (start >= L) return;
  const int n_keys = min(C, L - start);
  const int h0 = kvh * p.group + hg * GT;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int seg = lane % LPK;
  const int slot = lane / LPK;
  const int P = 1 << p.page_log2;

  // Page ids of the chunk.
  const int first_page = start >> p.page_log2;
  const int n_pages = ((start + n_keys - 1) >> p.page_log2) - first_page + 1;
  for (int i = tid; i < n_pages; i += kThreads)
    page_lds[i] = p.block_table[(size_t)b * p.max_pages + first_page + i];

  // This lane's segment of the GT queries.
  uint32_t qw[GT][4];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    const uint4 v = ld16(p.q + (((size_t)b * p.num_q_heads + h0 + h) * D + seg * EPL) * EB);
    qw[h][0] = v.x; qw[h][1] = v.y; qw[h][2] = v.z; qw[h][3] = v.w;
  }
  __syncthreads();

  const size_t head_stride = (size_t)P * D * EB;                 // one (page, head) tile
  const size_t page_stride = head_stride * p.num_kv_heads;
  auto row_ptr = [&](const uint8_t* base, int jl) -> const uint8_t* {
    const int j = start + jl;
    const int pg = page_lds[(j >> p.page_log2) - first_page];
    return base + (size_t)pg * page_stride + kvh * head_stride +
           (size_t)(j & (P - 1)) * D * EB + seg * 16;
  };

  // ---- phase 1: logits ----------------------------------------------------
  for (int kb = 0; kb < n_keys; kb += KPI * kUnroll) {
    uint4 kr[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int jl = kb + u * KPI + wave * KPW + slot;
      kr[u] = jl < n_keys ? ld16(row_ptr(p.k_pages, jl)) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int jl = kb + u * KPI + wave * KPW + slot;
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
      if (jl < n_keys) {
#pragma unroll
        for (int h = 0; h < GT; ++h)
          if (seg == h) s_lds[h * C + jl] = part[h] * p.scale;
      }
    }
  }
  __syncthreads();

  // ---- phase 2: chunk max, raw logits out, exp and chunk sum --------------
  for (int h = wave; h < GT; h += kWaves) {
    float* row = s_lds + h * C;
    float m = kNegInf;
    for (int i = lane; i < n_keys; i += kWave) m = fmaxf(m, row[i]);
    m = wave_max(m);
    const float ms = m * kLog2e;
    float* lg = WRITE_LOGITS ? p.logits + ((size_t)b * p.num_q_heads + h0 + h) * p.logits_stride + start
                             : nullptr;
    float l = 0.f;
    for (int i = lane; i < n_keys; i += kWave) {
      const float s = row[i];
      if constexpr (WRITE_LOGITS) lg[i] = s;
      const float e = exp2_hw(fmaf(s, kLog2e, -ms));
      row[i] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) ml_lds[h] = make_float2(m, l);
  }
  __syncthreads();

  const size_t ml_base = ((size_t)b * p.num_q_heads + h0) * p.n_chunks + chunk_id;
  if constexpr (!HAS_V) {
    if (tid < GT) p.part_ml[ml_base + (size_t)tid * p.n_chunks] = ml_lds[tid];
    return;
  } else {
    // ---- phase 3: P.V ------------------------------------------------------
    float acc[GT][EPL];
#pragma unroll
    for (int h = 0; h < GT; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;

    for (int kb = 0; kb < n_keys; kb += KPI * kUnroll) {
      uint4 vr[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int jl = kb + u * KPI + wave * KPW + slot;
        vr[u] = jl < n_keys ? ld16(row_ptr(p.v_pages, jl)) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int jl = kb + u * KPI + wave * KPW + slot;
        if (jl < n_keys) {
          float v[EPL];
          if constexpr (BF16) {
            v[0] = bf16lo(vr[u].x); v[1] = bf16hi(vr[u].x);
            v[2] = bf16lo(vr[u].y); v[3] = bf16hi(vr[u].y);
            v[4] = bf16lo(vr[u].z); v[5] = bf16hi(vr[u].z);
            v[6] = bf16lo(vr[u].w); v[7] = bf16hi(vr[u].w);
          } else {
            v[0] = __uint_as_float(vr[u].x); v[1] = __uint_as_float(vr[u].y);
            v[2] = __uint_as_float(vr[u].z); v[3] = __uint_as_float(vr[u].w);
          }
#pragma unroll
          for (int h = 0; h < GT; ++h) {
            const float pj = s_lds[h * C + jl];
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pj, v[e], acc[h][e]);
          }
        }
      }
    }
    // Sum over the key slots of the wave (lanes sharing a segment).
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
        for (int e = 0; e < EPL; ++e) red[(wave * GT + h) * D + seg * EPL + e] = acc[h][e];
    }
    __syncthreads();
    for (int idx = tid; idx < GT * D; idx += kThreads) {
      float o = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) o += red[w * GT * D + idx];
      const int h = idx / D, d = idx % D;
      p.part_o[((ml_base + (size_t)h * p.n_chunks)) * D + d] = o;
    }
    if (tid < GT) p.part_ml[ml_base + (size_t)tid * p.n_chunks] = ml_lds[tid];
  }
}

// ---- combine ----------------------------------------------------------------
struct CombineParams {
  const int32_t* seq_lens;
  const float* part_o;
  const float2* part_ml;
  float* out;       // [B][Hq][D] or null
  float* lse;       // [B][Hq] or null
  float* lse_ws;    // [B][Hq]
  int num_q_heads, chunk, n_chunks, D;
};

template <bool HAS_V>
__global__ __launch_bounds__(128) void decode_combine(CombineParams p) {
  const int bh = blockIdx.x;
  const int b = bh / p.num_q_heads;
  const int L = p.seq_lens[b];
  const int nc = (L + p.chunk - 1) / p.chunk;
  const float2* ml = p.part_ml + (size_t)bh * p.n_chunks;
  float M = kNegInf;
  for (int c = 0; c < nc; ++c) M = fmaxf(M, ml[c].x);
  const float Ms = M * kLog2e;
  float l = 0.f;
  for (int c = 0; c < nc; ++c) l += ml[c].y * exp2_hw(fmaf(ml[c].x, kLog2e, -Ms));
  if constexpr (HAS_V) {
    const int d = threadIdx.x;
    if (p.out && d < p.D) {
      const float* po = p.part_o + (size_t)bh * p.n_chunks * p.D + d;
      float o = 0.f;
      for (int c = 0; c < nc; ++c) o = fmaf(exp2_hw(fmaf(ml[c].x, kLog2e, -Ms)), po[(size_t)c * p.D], o);
      p.out[(size_t)bh * p.D + d] = o / l;
    }
  }
  if (threadIdx.x == 0) {
    const float v = M + log2_hw(l) * kLn2;
    p.lse_ws[bh] = v;
    if (p.lse) p.lse[bh] = v;
  }
}

// ---- normalise + accumulate ------------------------------------------------
struct FinalizeParams {
  const int32_t* seq_lens;
  const float* logits;  // [B][Hq][logits_stride]
  int64_t logits_stride;
  float* probs;         // [B][Hq][probs_stride] or null (may alias logits)
  int64_t probs_stride;
  const float* lse_ws;  // [B][Hq]
  float* cum;           // [B][Hkv][cum_stride] or null
  int64_t cum_stride;
  float decay;
  int num_q_heads, num_kv_heads, group, keys_per_block;
};

constexpr int kFinThreads = 256;

__global__ __launch_bounds__(kFinThreads) void decode_finalize(FinalizeParams p) {
  const int b = blockIdx.z;
  const int c = blockIdx.y;
  const int L = p.seq_lens[b];
  const int start = blockIdx.x * p.keys_per_block;
  if (start >= L) return;
  const int end = min(L, start + p.keys_per_block);
  const int h0 = c * p.group;
  for (int j = start + threadIdx.x; j < end; j += kFinThreads) {
    float acc = 0.f;
    for (int g = 0; g < p.group; ++g) {
      const size_t bh = (size_t)b * p.num_q_heads + h0 + g;
      const float s = p.logits[bh * p.logits_stride + j];
      const float e = exp2_hw((s - p.lse_ws[bh]) * kLog2e);
      if (p.probs) p.probs[bh * p.probs_stride + j] = e;
      acc += e;
    }
    if (p.cum) {
      float* cp = p.cum + ((size_t)b * p.num_kv_heads + c) * p.cum_stride + j;
      *cp = fmaf(p.decay, *cp, acc);
    }
  }
}

template <bool BF16, int D, int GT, bool HAS_V, bool WL>
hipError_t launch_partial_t(const PartialParams& pp, dim3 grid, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((decode_partial<BF16, D, GT, HAS_V, WL>), grid, dim3(kThreads), lds, s, pp);
  return hipGetLastError();
}

template <bool BF16, int D, int GT>
hipError_t launch_partial_g(const PartialParams& pp, bool has_v, bool wl, dim3 grid, size_t lds,
                            hipStream_t s) {
  if (has_v) {
    return wl ? launch_partial_t<BF16, D, GT, true, true>(pp, grid, lds, s)
              : launch_partial_t<BF16, D, GT, true, false>(pp, grid, lds, s);
  }
  return wl ? launch_partial_t<BF16, D, GT, false, true>(pp, grid, lds, s)
            : launch_partial_t<BF16, D, GT, false, false>(pp, grid, lds, s);
}

template <bool BF16, int D>
hipError_t launch_partial_d(const PartialParams& pp, int gt, bool has_v, bool wl, dim3 grid,
                            size_t lds, hipStream_t s) {
  switch (gt) {
    case 1: return launch_partial_g<BF16, D, 1>(pp, has_v, wl, grid, lds, s);
    case 2: return launch_partial_g<BF16, D, 2>(pp, has_v, wl, grid, lds, s);
    case 4: return launch_partial_g<BF16, D, 4>(pp, has_v, wl, grid, lds, s);
    case 8: return launch_partial_g<BF16, D, 8>(pp, has_v, wl, grid, lds, s);
    default: return hipErrorInvalidValue;
  }
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

DecodePlan plan_decode(int num_seqs, int num_kv_heads, int num_q_heads, int head_dim,
                       int max_seq_len, bool need_scratch) {
  DecodePlan pl{};
  const int G = num_q_heads / num_kv_heads;
  pl.gt = G >= 8 ? 8 : G;
  pl.hgroups = G / pl.gt;
  // Largest chunk (<= 512 keys) that still gives the grid >= 2048 workgroups,
  // never below 64 keys.
  int chunk = 512;
  while (chunk > 64) {
    const long long wgs = (long long)num_seqs * num_kv_heads * pl.hgroups *
                          ((max_seq_len + chunk - 1) / chunk);
    if (wgs >= 2048) break;
    chunk /= 2;
  }
  pl.chunk = chunk;
  pl.n_chunks = (max_seq_len + chunk - 1) / chunk;
  const size_t bh = (size_t)num_seqs * num_q_heads;
  pl.part_o_bytes = align256(bh * pl.n_chunks * head_dim * sizeof(float));
  pl.part_ml_bytes = align256(bh * pl.n_chunks * sizeof(float2));
  pl.lse_bytes = align256(bh * sizeof(float));
  pl.scratch_bytes = need_scratch ? align256(bh * (size_t)max_seq_len * sizeof(float)) : 0;
  pl.total_bytes = pl.part_o_bytes + pl.part_ml_bytes + pl.lse_bytes + pl.scratch_bytes;
  return pl;
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& pl, hipStream_t stream) {
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  float* part_o = reinterpret_cast<float*>(ws);
  float2* part_ml = reinterpret_cast<float2*>(ws + pl.part_o_bytes);
  float* lse_ws = reinterpret_cast<float*>(ws + pl.part_o_bytes + pl.part_ml_bytes);
  float* scratch = reinterpret_cast<float*>(ws + pl.part_o_bytes + pl.part_ml_bytes + pl.lse_bytes);

  const bool use_v = a.v_pages != nullptr && a.out != nullptr;
  const bool need_norm = !a.emit_logits && (a.probs != nullptr || a.cum != nullptr);
  float* logits = nullptr;
  int64_t logits_stride = 0;
  if (a.probs) {
    logits = a.probs;
    logits_stride = a.probs_stride;
  } else if (need_norm) {
    logits = scratch;
    logits_stride = a.max_seq_len;
  }

  PartialParams pp{};
  pp.k_pages = static_cast<const uint8_t*>(a.k_pages);
  pp.v_pages = static_cast<const uint8_t*>(a.v_pages);
  pp.block_table = a.block_table;
  pp.seq_lens = a.seq_lens;
  pp.q = static_cast<const uint8_t*>(a.q);
  pp.logits = logits;
  pp.logits_stride = logits_stride;
  pp.part_o = part_o;
  pp.part_ml = part_ml;
  pp.num_kv_heads = a.num_kv_heads;
  pp.num_q_heads = a.num_q_heads;
  pp.group = a.num_q_heads / a.num_kv_heads;
  pp.hgroups = pl.hgroups;
  pp.page_log2 = __builtin_ctz((unsigned)a.page_size);
  pp.max_pages = a.max_pages;
  pp.chunk = pl.chunk;
  pp.n_chunks = pl.n_chunks;
  pp.scale = a.scale;

  const dim3 grid(pl.n_chunks, a.num_kv_heads * pl.hgroups, a.num_seqs);
  const size_t lds = (size_t)pl.gt * pl.chunk * sizeof(float) +
                     (size_t)kWaves * pl.gt * a.head_dim * sizeof(float) + pl.gt * sizeof(float2) +
                     ((size_t)pl.chunk / 16 + 2) * sizeof(int);
  const bool wl = logits != nullptr;
  hipError_t e;
  if (a.bf16) {
    e = a.head_dim == 128 ? launch_partial_d<true, 128>(pp, pl.gt, use_v, wl, grid, lds, stream)
                          : launch_partial_d<true, 64>(pp, pl.gt, use_v, wl, grid, lds, stream);
  } else {
    e = a.head_dim == 128 ? launch_partial_d<false, 128>(pp, pl.gt, use_v, wl, grid, lds, stream)
                          : launch_partial_d<false, 64>(pp, pl.gt, use_v, wl, grid, lds, stream);
  }
  if (e != hipSuccess) return e;

  // The combine is needed for out, lse, or the normalisation.
  if (a.out || a.lse || need_norm) {
    {
      CombineParams cp{};
      cp.seq_lens = a.seq_lens;
      cp.part_o = part_o;
      cp.part_ml = part_ml;
      cp.out = use_v ? a.out : nullptr;
      cp.lse = a.lse;
      cp.lse_ws = lse_ws;
      cp.num_q_heads = a.num_q_heads;
      cp.chunk = pl.chunk;
      cp.n_chunks = pl.n_chunks;
      cp.D = a.head_dim;
      const dim3 cgrid(a.num_seqs * a.num_q_heads);
      if (use_v)
        hipLaunchKernelGGL(decode_combine<true>, cgrid, dim3(a.head_dim), 0, stream, cp);
      else
        hipLaunchKernelGGL(decode_combine<false>, cgrid, dim3(64), 0, stream, cp);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }

  if (need_norm) {
    FinalizeParams fp{};
    fp.seq_lens = a.seq_lens;
    fp.logits = logits;
    fp.logits_stride = logits_stride;
    fp.probs = a.probs;
    fp.probs_stride = a.probs_stride;
    fp.lse_ws = lse_ws;
    fp.cum = a.cum;
    fp.cum_stride = a.cum_stride;
    fp.decay = a.decay;
    fp.num_q_heads = a.num_q_heads;
    fp.num_kv_heads = a.num_kv_heads;
    fp.group = a.num_q_heads / a.num_kv_heads;
    fp.keys_per_block = 1024;
    const dim3 fgrid((a.max_seq_len + fp.keys_per_block - 1) / fp.keys_per_block, a.num_kv_heads,
                     a.num_seqs);
    hipLaunchKernelGGL(decode_finalize, fgrid, dim3(kFinThreads), 0, stream, fp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kvsel
