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

// Tuning knobs (compile-time).
#ifndef KVSEL_NT_KV
#define KVSEL_NT_KV 1      // stream K/V with non-temporal loads
#endif
#ifndef KVSEL_NT_K_QK
#define KVSEL_NT_K_QK 1    // 1: the MFMA K-fragment loads non-temporal too (with whole-line loads
                           // no line is read twice; with half-line loads cached reads let the
                           // second half hit)
#endif
#ifndef KVSEL_MAX_CHUNK
#define KVSEL_MAX_CHUNK 1024 // keys per split-K chunk (multiple of 64)
#endif
#ifndef KVSEL_FIXED_CHUNK
#define KVSEL_FIXED_CHUNK 0  // >0: always use this chunk (multiple of 64, <= KVSEL_MAX_CHUNK)
#endif
#ifndef KVSEL_MIN_WGS
#define KVSEL_MIN_WGS 1024   // shrink the chunk until the grid has this many workgroups
#endif
#ifndef KVSEL_PV_VU
#define KVSEL_PV_VU 0        // >0: P.V value loads per lane per batch (double-buffered) for every group width
#endif
#ifndef KVSEL_QK_DB
#define KVSEL_QK_DB 0        // 1: double-buffer the K batches of the QK phase
#endif
#ifndef KVSEL_QK_BATCH
#define KVSEL_QK_BATCH 0     // >0: issue the K loads of this many tiles before their MFMAs (0: per kernel)
#endif
#ifndef KVSEL_WAVES_PER_EU
#define KVSEL_WAVES_PER_EU 0 // >0: occupancy hint for the kernels with P.V (0: per kernel)
#endif
#ifndef KVSEL_COOP_NORM
#define KVSEL_COOP_NORM 1  // normalise probabilities inside the split-K pass (bf16, G <= 8)
#endif
#ifndef KVSEL_NT_PROBS
#define KVSEL_NT_PROBS 1   // write final probabilities with non-temporal stores
#endif
#ifndef KVSEL_NT_CUM
#define KVSEL_NT_CUM 0     // 1: write the updated cum with non-temporal stores
#endif
#ifndef KVSEL_K_LINES
#define KVSEL_K_LINES 1    // 1: K fragments loaded as whole 128-byte lines, then traded between lanes
#endif

__device__ __forceinline__ uint4 ld_kv(const void* ptr) {
#if KVSEL_NT_KV
  return ld16_stream(ptr);
#else
  return ld16(ptr);
#endif
}

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
  int num_rows;                  // B * H_kv
  // In-kernel normalisation (rows of one (sequence, KV head)):
  unsigned long long* lse_post;  // [B][Hq][n_chunks][2] chunk lse tagged with epoch / ~epoch
  uint32_t* chunk_flag;          // [B][H_kv][n_chunks] 1 when the chunk fell back, else 0
  uint32_t epoch;
  unsigned long long wait_ticks; // bound of the wait for the row's posts, in wall-clock ticks
  float* probs;                  // final probabilities [B][Hq][probs_stride] or null
  int64_t probs_stride;
  float* raw;                    // fallback target for chunk-relative exp values
  int64_t raw_stride;
  float* cum;                    // [B][H_kv][cum_stride] or null
  int64_t cum_stride;
  float decay;
  // Block aggregates of the updated cum (blk_bs > 0): max and mean over the
  // valid positions of each block of blk_bs, per (sequence, KV head).
  int blk_bs;
  float* blk_max;                // [b * blk_seq_stride + kvh * blk_head_stride + block] or null
  float* blk_mean;
  int64_t blk_head_stride, blk_seq_stride;
  float* lse_out;                // [B][Hq] or null: written by the first chunk of a completed row
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

// ---- bf16 partial pass with the QK^T tile on the matrix cores ---------------
// One 16-key tile of one KV head against the (up to 16) query heads of its
// group is the product K_tile (16 x d) . Q^T (d x 16): v_mfma_f32_16x16x32_bf16
// with keys as rows and heads as columns.  bf16 x bf16 products are exact in
// fp32, so the logits equal the VALU dot products up to summation order.
// Every logit lands on exactly one lane (lane = head + 16 * (key / 4),
// register = key % 4), so the softmax arithmetic is done once per (key, head).
// P.V stays on the vector ALUs: lanes own 8 dims of a value row and read the
// group's probabilities of that key from a key-major LDS tile.
// Occupancy of the kernels with P.V: four workgroups (16 waves) per CU.
// LDS allows it at 1024-key chunks (the [C][GT] probability tile, 32 KB at
// G = 8, plus one [GT][D] reduction tile); registers (<= 128) need one K tile
// per load batch and two value loads per lane at G = 8 with the normalisation,
// two K tiles and four value loads below G = 8.  D = 64 at G = 8 does not fit
// 128 registers without spills and keeps three waves per SIMD.
template <int D, int GT, bool HAS_V>
constexpr bool kDecodeWide64 = HAS_V && D == 64 && GT >= 8;
template <int D, int GT, bool HAS_V>
constexpr int kDecodeWaves = KVSEL_WAVES_PER_EU > 0 && HAS_V ? KVSEL_WAVES_PER_EU : kDecodeWide64<D, GT, HAS_V> ? 3 : 4;

template <int D, int GT, bool HAS_V, bool WRITE_LOGITS, bool COOP>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kDecodeWaves<D, GT, HAS_V>)))
void decode_partial_mfma(PartialParams p) {
  constexpr int NU = D / 32;                 // MFMA k-steps (32 dims each)
  constexpr int EPL = 8;                     // P.V: dims per lane
  constexpr int LPK = D / EPL;               // P.V: lanes per value row
  constexpr int KPW = kWave / LPK;           // P.V: keys per wave per load
  constexpr int KPI = kWaves * KPW;          // P.V: keys per workgroup per load
  // P.V: value loads per lane per batch, as many as the register budget of
  // the group width allows without spilling.
  constexpr bool W64 = kDecodeWide64<D, GT, HAS_V>;
  constexpr int VU = KVSEL_PV_VU > 0 ? KVSEL_PV_VU : GT >= 8 && COOP && !W64 ? 2 : 4;
  // K tiles per load batch
  constexpr int QB = KVSEL_QK_BATCH > 0 ? KVSEL_QK_BATCH : !HAS_V || W64 ? 4 : GT >= 8 ? 1 : 2;

  extern __shared__ __align__(16) float smem[];
  const int C = p.chunk;
  float* p_lds = smem;                               // [C][GT] logits, then exp(s - m)
  // [GT][D] reduction tile of P.V; then [GT][n_chunks] posts of the row
  float* red = smem + C * GT;
  float* wstat = red + GT * (COOP ? max(D, p.n_chunks) : D);           // [2][kWaves][16]
  float2* ml_lds = reinterpret_cast<float2*>(wstat + 2 * kWaves * 16);  // [GT]
  int* page_lds = reinterpret_cast<int*>(ml_lds + GT);                  // [C/16 + 2]

  int chunk_id, kvh, hg, b;
  if constexpr (COOP) {
    // 1-D grid over the chunks that exist: sequence-major, then KV head,
    // then chunk, with the chunks past each sequence's end left out.  Every
    // workgroup recomputes the map from seq_lens (a scan by wave 0).  Rows
    // of the same length are thus dispatched as one burst spread over all
    // XCDs, so a row's chunks run together and the wait for the row's posts
    // stays short; surplus workgroups at the end of the grid exit.
    int* map = reinterpret_cast<int*>(wstat);
    const int w = blockIdx.x;
    const int lane0 = threadIdx.x % kWave;
    const int nseq = p.num_rows / p.num_kv_heads;
    if (threadIdx.x < kWave) {
      if (lane0 == 0) map[0] = -1;
      int base = 0;
      for (int b0 = 0; b0 < nseq; b0 += kWave) {
        const int bb = b0 + lane0;
        const int cnt = bb < nseq ? p.num_kv_heads * ((p.seq_lens[bb] + C - 1) / C) : 0;
        int incl = cnt;
#pragma unroll
        for (int off = 1; off < kWave; off *= 2) {
          const int t = __shfl_up(incl, off, kWave);
          if (lane0 >= off) incl += t;
        }
        const int lo = base + incl - cnt;
        if (cnt > 0 && w >= lo && w < lo + cnt) {
          const int ncb = cnt / p.num_kv_heads;
          map[0] = bb;
          map[1] = (w - lo) / ncb;
          map[2] = (w - lo) % ncb;
        }
        base += __shfl(incl, kWave - 1, kWave);
        if (w < base) break;
      }
    }
    __syncthreads();
    if (map[0] < 0) return;
    b = map[0];
    kvh = map[1];
    chunk_id = map[2];
    hg = 0;
    __syncthreads();   // map lives in wstat, which phase 2 reuses
  } else {
    chunk_id = blockIdx.x;
    kvh = blockIdx.y / p.hgroups;
    hg = blockIdx.y % p.hgroups;
    b = blockIdx.z;
  }
  const int L = p.seq_lens[b];
  const int start = chunk_id * C;
  if (start >= L) return;
  const int n_keys = min(C, L - start);
  const int h0 = kvh * p.group + hg * GT;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int col = lane & 15;   // A row (key slot) and B column (head slot)
  const int grp = lane >> 4;   // k-group of the operands, row-quad of the result
  const int P = 1 << p.page_log2;

  const int first_page = start >> p.page_log2;
  const int n_pages = ((start + n_keys - 1) >> p.page_log2) - first_page + 1;
  for (int i = tid; i < n_pages; i += kThreads)
    page_lds[i] = p.block_table[(size_t)b * p.max_pages + first_page + i];

  // B operand (Q^T): column = head slot, k = dims u*32 + grp*8 .. +8.
  bf16x8 qb[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    uint4 w = make_uint4(0, 0, 0, 0);
    if (col < GT) w = ld16(p.q + (((size_t)b * p.num_q_heads + h0 + col) * D + u * 32 + grp * 8) * 2);
    qb[u] = __builtin_bit_cast(bf16x8, w);
  }
  __syncthreads();

  const size_t head_stride = (size_t)P * D * 2;
  const size_t page_stride = head_stride * p.num_kv_heads;
  auto row_base = [&](const uint8_t* base, int jl) -> const uint8_t* {
    const int j = start + jl;
    const int pg = page_lds[(j >> p.page_log2) - first_page];
    return base + (size_t)pg * page_stride + kvh * head_stride + (size_t)(j & (P - 1)) * D * 2;
  };

  // ---- phase 1: logits, tile by tile, into LDS (and out to global) --------
  // A wave owns a contiguous range of 16-key tiles.  K loads are issued a
  // batch of QB tiles at a time, every address clamped to a valid key so
  // the loads are unconditional; keys past the end are masked to -inf.
  const int per_wave = C / kWaves;       // multiple of 16
  const int nt = per_wave / 16;
  const int wbase = wave * per_wave;
  float* lg = nullptr;
  bool lg_vec = false;
  if constexpr (WRITE_LOGITS) {
    lg = p.logits + ((size_t)b * p.num_q_heads + h0 + min(col, GT - 1)) * p.logits_stride + start;
    lg_vec = (p.logits_stride & 3) == 0 && (reinterpret_cast<uintptr_t>(p.logits) & 15) == 0 &&
             n_keys == C;
  }
  float mrun = kNegInf;
  auto load_k = [&](bf16x8 (&kb)[QB][NU], int t0) {
#pragma unroll
    for (int t = 0; t < QB; ++t) {
      if constexpr (KVSEL_K_LINES) {
        const int key = wbase + min(t0 + t, nt - 1) * 16 + (col & 7);
        const int sg = (grp + 4 * (col >> 3)) * 16;
        const uint8_t* ra = row_base(p.k_pages, min(key, n_keys - 1)) + sg;
        const uint8_t* rb = row_base(p.k_pages, min(key + 8, n_keys - 1)) + sg;
#pragma unroll
        for (int v = 0; v < NU / 2; ++v) {
          kb[t][2 * v] = __builtin_bit_cast(bf16x8, KVSEL_NT_K_QK ? ld_kv(ra + v * 128) : ld16(ra + v * 128));
          kb[t][2 * v + 1] = __builtin_bit_cast(bf16x8, KVSEL_NT_K_QK ? ld_kv(rb + v * 128) : ld16(rb + v * 128));
        }
      } else {
        const int key = min(wbase + min(t0 + t, nt - 1) * 16 + col, n_keys - 1);
        const uint8_t* rp = row_base(p.k_pages, key) + grp * 16;
#pragma unroll
        for (int u = 0; u < NU; ++u) kb[t][u] = __builtin_bit_cast(bf16x8, KVSEL_NT_K_QK ? ld_kv(rp + u * 64) : ld16(rp + u * 64));
      }
    }
  };
  auto tile_k = [&](bf16x8 (&kb)[QB][NU], int t0) {
#pragma unroll
    for (int t = 0; t < QB; ++t) {
      if (t0 + t < nt) {
        if constexpr (KVSEL_K_LINES) {
#pragma unroll
          for (int v = 0; v < NU / 2; ++v) k_line_exchange(kb[t][2 * v], kb[t][2 * v + 1], col < 8);
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < NU; ++u)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[t][u], qb[u], acc, 0, 0, 0);
        const int k0 = wbase + (t0 + t) * 16 + grp * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = (k0 + i < n_keys) ? acc[i] * p.scale : kNegInf;
        mrun = fmaxf(mrun, fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3])));
        if (col < GT) {
#pragma unroll
          for (int i = 0; i < 4; ++i) p_lds[(k0 + i) * GT + col] = acc[i];
          if constexpr (WRITE_LOGITS) {
            if (lg_vec) {
              *reinterpret_cast<float4*>(lg + k0) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (k0 + i < n_keys) lg[k0 + i] = acc[i];
            }
          }
        }
      }
    }
  };
  if constexpr (KVSEL_QK_DB && HAS_V) {   // the K-only variants have no registers to spare
    // two batches in flight: the next batch's K loads go out before the
    // current batch's MFMAs (past the last tile the loads are clamped to it)
    bf16x8 ka[QB][NU], kc[QB][NU];
    load_k(ka, 0);
    for (int t0 = 0; t0 < nt; t0 += 2 * QB) {
      load_k(kc, t0 + QB);
      tile_k(ka, t0);
      load_k(ka, t0 + 2 * QB);
      tile_k(kc, t0 + QB);
    }
  } else {
    for (int t0 = 0; t0 < nt; t0 += QB) {
      bf16x8 kb[QB][NU];
      load_k(kb, t0);
      __builtin_amdgcn_sched_barrier(0);
      tile_k(kb, t0);
    }
  }

  // P.V lane mapping: a lane owns 8 dims (one 16-byte segment) of a value
  // row.  The first V batch is issued here so that it is in flight while the
  // softmax of phase 2 runs.
  const int seg = lane % LPK;
  const int slot = lane / LPK;
  // Clamped, unconditional loads; keys past the end get p = 0.
  auto load_batch = [&](uint4 (&vr)[VU], int kb) {
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int jl = min(kb + u * KPI + wave * KPW + slot, n_keys - 1);
      vr[u] = ld_kv(row_base(p.v_pages, jl) + seg * 16);
    }
  };
  [[maybe_unused]] uint4 va[VU];
  if constexpr (HAS_V) load_batch(va, 0);

  // ---- phase 2: chunk max and sum of exp per head, p = exp(s - m) in LDS ---
  mrun = fmaxf(mrun, __shfl_xor(mrun, 16, kWave));
  mrun = fmaxf(mrun, __shfl_xor(mrun, 32, kWave));
  if (grp == 0) wstat[wave * 16 + col] = mrun;
  __syncthreads();
  {
    // A thread always meets the same head: element idx = tid + 256 i of the
    // [C][GT] tile has head idx % GT = tid % GT.
    const int hh = tid % GT;
    const float m = fmaxf(fmaxf(wstat[hh], wstat[16 + hh]), fmaxf(wstat[32 + hh], wstat[48 + hh]));
    const float ms = m * kLog2e;
    float l = 0.f;
    for (int idx = tid; idx < C * GT; idx += kThreads) {
      const float e = exp2_hw(fmaf(p_lds[idx], kLog2e, -ms));
      p_lds[idx] = e;
      l += e;
    }
#pragma unroll
    for (int off = GT; off < kWave; off *= 2) l += __shfl_xor(l, off, kWave);
    if (lane < GT) wstat[64 + wave * 16 + lane] = l;
    __syncthreads();
    if (tid < GT)
      ml_lds[tid] = make_float2(m, (wstat[64 + tid] + wstat[80 + tid]) + (wstat[96 + tid] + wstat[112 + tid]));
    __syncthreads();
  }

  const size_t ml_base = ((size_t)b * p.num_q_heads + h0) * p.n_chunks + chunk_id;
  const size_t row = (size_t)b * p.num_kv_heads + kvh;   // COOP runs with hgroups == 1
  if constexpr (COOP) {
    // Post this chunk's log-sum-exp per head as two 64-bit words, the value
    // tagged once with the call's epoch and once with its complement.  Each
    // word validates itself, so neither side needs a fence (relaxed
    // agent-scope stores, read back with relaxed loads).  The combine zeroes
    // the posts after the pass, so a workspace that served an earlier call
    // holds none (a graph replays one epoch), and junk in a fresh workspace
    // passes the check with probability 2^-64.
    if (tid < 2 * GT) {
      const int h = tid >> 1;
      const float2 ml = ml_lds[h];
      const float lse_c = ml.x + log2_hw(ml.y) * kLn2;
      const uint32_t tag = (tid & 1) ? ~p.epoch : p.epoch;
      const unsigned long long w = ((unsigned long long)tag << 32) | __float_as_uint(lse_c);
      __hip_atomic_store(p.lse_post + 2 * (ml_base + (size_t)h * p.n_chunks) + (tid & 1), w, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // Row-wide state of the in-kernel normalisation.  A thread owns 4
  // consecutive keys of the chunk (16-byte accesses when the rows allow).
  // The chunk's slice of cum is read here, ahead of P.V, so no latency is
  // left for the end (probs and cum may alias, so the compiler could not
  // hoist it itself).
  constexpr int JPT = (KVSEL_MAX_CHUNK + 4 * kThreads - 1) / (4 * kThreads);
  const int nc = (L + C - 1) / C;
  const int nw = GT * nc;
  const unsigned long long* post = p.lse_post + 2 * ((size_t)b * p.num_q_heads + h0) * p.n_chunks;
  // Post i = (head, chunk) of the row: the two tagged words are loaded, and
  // validated separately so the loads can be issued well ahead of the check.
  // An invalid pair reads as 0, whose high word never equals the tag.
  auto post_load = [&](int i, unsigned long long& w0, unsigned long long& w1) {
    const int h = i / nc, c = i - h * nc;
    const unsigned long long* w = post + 2 * ((size_t)h * p.n_chunks + c);
    w0 = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    w1 = __hip_atomic_load(w + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  auto post_check = [&](unsigned long long w0, unsigned long long w1) -> unsigned long long {
    const bool valid = (uint32_t)(w0 >> 32) == p.epoch && (uint32_t)(w1 >> 32) == ~p.epoch &&
                       (uint32_t)w0 == (uint32_t)w1;
    return valid ? w0 : 0ull;
  };
  auto post_word = [&](int i) -> unsigned long long {
    unsigned long long w0, w1;
    post_load(i, w0, w1);
    return post_check(w0, w1);
  };
  float* cum_row = (COOP && p.cum) ? p.cum + row * p.cum_stride + start : nullptr;
  float* prow = (COOP && p.probs) ? p.probs + ((size_t)b * p.num_q_heads + h0) * p.probs_stride + start : nullptr;
  const bool cum_vec = ((reinterpret_cast<uintptr_t>(cum_row) | ((uintptr_t)p.cum_stride * 4)) & 15) == 0;
  const bool probs_vec = ((reinterpret_cast<uintptr_t>(prow) | ((uintptr_t)p.probs_stride * 4)) & 15) == 0;
  [[maybe_unused]] float4 cpre[JPT];
  [[maybe_unused]] unsigned long long w_first = 0, w_first1 = 0;
  if constexpr (COOP) {
#pragma unroll
    for (int i = 0; i < JPT; ++i) {
      const int j0 = 4 * (tid + i * kThreads);
      float4 c = make_float4(0.f, 0.f, 0.f, 0.f);
      if (cum_row && j0 < n_keys) {
        if (cum_vec && j0 + 3 < n_keys) {
          c = *reinterpret_cast<const float4*>(cum_row + j0);
        } else {
          c.x = cum_row[j0];
          if (j0 + 1 < n_keys) c.y = cum_row[j0 + 1];
          if (j0 + 2 < n_keys) c.z = cum_row[j0 + 2];
          if (j0 + 3 < n_keys) c.w = cum_row[j0 + 3];
        }
      }
      cpre[i] = c;
    }
  }
  constexpr int kNO = (GT * D + kThreads - 1) / kThreads;   // partial outputs per thread
  [[maybe_unused]] float ov[kNO];
  if constexpr (!HAS_V) {
    if (tid < GT) p.part_ml[ml_base + (size_t)tid * p.n_chunks] = ml_lds[tid];
    if constexpr (!COOP) return;
  } else {
    // ---- phase 3: P.V on the vector ALUs -----------------------------------
    float acc[GT][EPL];
#pragma unroll
    for (int h = 0; h < GT; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;

    auto fma_batch = [&](const uint4 (&vr)[VU], int kb) {
#pragma unroll
      for (int u = 0; u < VU; ++u) {
        const int jr = kb + u * KPI + wave * KPW + slot;
        const bool valid = jr < n_keys;
        const int jl = min(jr, n_keys - 1);
        {
          float v[EPL];
          v[0] = bf16lo(vr[u].x); v[1] = bf16hi(vr[u].x);
          v[2] = bf16lo(vr[u].y); v[3] = bf16hi(vr[u].y);
          v[4] = bf16lo(vr[u].z); v[5] = bf16hi(vr[u].z);
          v[6] = bf16lo(vr[u].w); v[7] = bf16hi(vr[u].w);
          float pj[GT];
          if constexpr (GT >= 4) {
#pragma unroll
            for (int h4 = 0; h4 < GT / 4; ++h4) {
              const float4 t4 = *reinterpret_cast<const float4*>(p_lds + jl * GT + 4 * h4);
              pj[4 * h4] = t4.x; pj[4 * h4 + 1] = t4.y; pj[4 * h4 + 2] = t4.z; pj[4 * h4 + 3] = t4.w;
            }
          } else {
#pragma unroll
            for (int h = 0; h < GT; ++h) pj[h] = p_lds[jl * GT + h];
          }
#pragma unroll
          for (int h = 0; h < GT; ++h) pj[h] = valid ? pj[h] : 0.f;
#pragma unroll
          for (int h = 0; h < GT; ++h)
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pj[h], v[e], acc[h][e]);
        }
      }
    };
    constexpr int STEP = KPI * VU;
    uint4 vb[VU];
    // The first poll of the row's posts is issued half way through P.V (the
    // other chunks posted long before), and checked after it.
    const int kb_poll = (n_keys / (4 * STEP)) * (2 * STEP);
    for (int kb = 0; kb < n_keys; kb += 2 * STEP) {
      if constexpr (COOP)
        if (kb == kb_poll && tid < nw) post_load(tid, w_first, w_first1);
      load_batch(vb, kb + STEP);
      fma_batch(va, kb);
      load_batch(va, kb + 2 * STEP);
      fma_batch(vb, kb + STEP);
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
    // The waves' sums meet in one [GT][D] tile: the last wave stores its
    // own, each earlier wave in turn adds its own (one tile rather than one
    // per wave is what keeps four workgroups per CU within the LDS).
#pragma unroll
    for (int w = kWaves - 1; w >= 0; --w) {
      if (wave == w && slot == 0) {
#pragma unroll
        for (int h = 0; h < GT; ++h) {
          float4* r = reinterpret_cast<float4*>(red + h * D + seg * EPL);
          float4 x0 = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
          float4 x1 = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
          if (w != kWaves - 1) {
            const float4 y0 = r[0], y1 = r[1];
            x0 = make_float4(y0.x + x0.x, y0.y + x0.y, y0.z + x0.z, y0.w + x0.w);
            x1 = make_float4(y1.x + x1.x, y1.y + x1.y, y1.z + x1.z, y1.w + x1.w);
          }
          r[0] = x0;
          r[1] = x1;
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < kNO; ++i) {
      const int idx = tid + i * kThreads;
      ov[i] = idx < GT * D ? red[idx] : 0.f;
      // Without in-kernel normalisation the partial output goes out as is;
      // with it, once the row's lse is known (phase 4).
      if (!COOP && idx < GT * D) p.part_o[((ml_base + (size_t)(idx / D) * p.n_chunks)) * D + idx % D] = ov[i];
    }
    if (tid < GT) p.part_ml[ml_base + (size_t)tid * p.n_chunks] = ml_lds[tid];
  }
  if constexpr (COOP) {
    // ---- phase 4: exact probabilities and cum, written once ---------------
    // Gather the posted lse of every chunk of the row (bounded wait); the
    // posts happen before P.V, so the first poll normally finds them all.
    float* lse_lds = red;                                     // [GT][nc], red is free again
    float* fac = wstat;                                       // [GT] exp(m_chunk - lse)
    __syncthreads();
    if constexpr (!HAS_V) {
      if (tid < nw) w_first = post_word(tid);
    } else {
      if (tid < nw) w_first = post_check(w_first, w_first1);
    }
    int miss0 = 0;
    if (tid < nw) {
      if ((uint32_t)(w_first >> 32) != p.epoch) miss0 = 1;
      else lse_lds[tid] = __uint_as_float((uint32_t)w_first);
    }
    for (int i = tid + kThreads; i < nw; i += kThreads) {   // rows of more than kThreads posts
      const unsigned long long w = post_word(i);
      if ((uint32_t)(w >> 32) != p.epoch) miss0 = 1;
      else lse_lds[i] = __uint_as_float((uint32_t)w);
    }
    bool ok = !__syncthreads_or(miss0);
    if (!ok && p.wait_ticks > 0) {
      // Poll again until the row is complete or wait_ticks of the constant
      // wall clock have passed.  Only thread 0's clock decides; it publishes
      // the decision in LDS before the barrier that every thread then reads
      // it after.  Two slots alternate, so the next write (after the next
      // barrier) never races the reads.  The slots sit in the dynamic area
      // (wstat past fac[GT]): a static LDS variable would shift the dynamic
      // area off its 16-byte alignment and split every float4 LDS access.
      int* expired = reinterpret_cast<int*>(wstat + 64);
      const unsigned long long t0 = (unsigned long long)wall_clock64();
      for (int it = 0; !ok; ++it) {
        if (tid == 0) expired[it & 1] = ((unsigned long long)wall_clock64() - t0) >= p.wait_ticks;
        __builtin_amdgcn_s_sleep(2);
        int miss = 0;
        for (int i = tid; i < nw; i += kThreads) {
          const unsigned long long w = post_word(i);
          if ((uint32_t)(w >> 32) != p.epoch) miss = 1;
          else lse_lds[i] = __uint_as_float((uint32_t)w);
        }
        ok = !__syncthreads_or(miss);
        if (!ok && expired[it & 1]) break;
      }
    }
    if (ok) {
      for (int h = wave; h < GT; h += kWaves) {
        float M = kNegInf;
        for (int c = lane; c < nc; c += kWave) M = fmaxf(M, lse_lds[h * nc + c]);
        M = wave_max(M);
        const float Ms = M * kLog2e;
        float l = 0.f;
        for (int c = lane; c < nc; c += kWave) l += exp2_hw(fmaf(lse_lds[h * nc + c], kLog2e, -Ms));
        l = wave_sum(l);
        const float lse = M + log2_hw(l) * kLn2;
        if (lane == 0) {
          fac[h] = exp2_hw((ml_lds[h].x - lse) * kLog2e);
          if (chunk_id == 0 && p.lse_out) p.lse_out[(size_t)b * p.num_q_heads + h0 + h] = lse;
        }
      }
      __syncthreads();
      if constexpr (HAS_V) {
        // The partial output already weighted by exp(m_chunk - lse): the
        // combine only sums the chunks of a completed row.
#pragma unroll
        for (int i = 0; i < kNO; ++i) {
          const int idx = tid + i * kThreads;
          if (idx < GT * D)
            p.part_o[((ml_base + (size_t)(idx / D) * p.n_chunks)) * D + idx % D] = ov[i] * fac[idx / D];
        }
      }
      float f[GT];
#pragma unroll
      for (int h = 0; h < GT; ++h) f[h] = fac[h];
#pragma unroll
      for (int i = 0; i < JPT; ++i) {
        const int j0 = 4 * (tid + i * kThreads);
        float bmax = kNegInf, bsum = 0.f;        // this thread's part of its block
        if (j0 < n_keys) {
          // p_lds[(j0 .. j0+3) * GT + h]: 4 GT contiguous floats
          float pv[4][GT];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            if constexpr (GT >= 4) {
#pragma unroll
              for (int h4 = 0; h4 < GT / 4; ++h4) {
                const float4 t4 = *reinterpret_cast<const float4*>(p_lds + (j0 + k) * GT + 4 * h4);
                pv[k][4 * h4] = t4.x * f[4 * h4];
                pv[k][4 * h4 + 1] = t4.y * f[4 * h4 + 1];
                pv[k][4 * h4 + 2] = t4.z * f[4 * h4 + 2];
                pv[k][4 * h4 + 3] = t4.w * f[4 * h4 + 3];
              }
            } else {
#pragma unroll
              for (int h = 0; h < GT; ++h) pv[k][h] = p_lds[(j0 + k) * GT + h] * f[h];
            }
          }
          const bool full = j0 + 3 < n_keys;
          if (prow) {
#pragma unroll
            for (int h = 0; h < GT; ++h) {
              float* dst = prow + (size_t)h * p.probs_stride + j0;
              if (probs_vec && full) {
                typedef float f32x4v __attribute__((ext_vector_type(4)));
                __builtin_nontemporal_store(f32x4v{pv[0][h], pv[1][h], pv[2][h], pv[3][h]},
                                            reinterpret_cast<f32x4v*>(dst));
              } else {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                  if (j0 + k < n_keys) dst[k] = pv[k][h];
              }
            }
          }
          if (cum_row) {
            float a[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              a[k] = 0.f;
#pragma unroll
              for (int h = 0; h < GT; ++h) a[k] += pv[k][h];
            }
            const float4 c = cpre[i];
            const float4 r = make_float4(fmaf(p.decay, c.x, a[0]), fmaf(p.decay, c.y, a[1]),
                                         fmaf(p.decay, c.z, a[2]), fmaf(p.decay, c.w, a[3]));
            if (cum_vec && full) {
              if constexpr (KVSEL_NT_CUM) {
                typedef float f32x4v __attribute__((ext_vector_type(4)));
                __builtin_nontemporal_store(f32x4v{r.x, r.y, r.z, r.w}, reinterpret_cast<f32x4v*>(cum_row + j0));
              } else {
                *reinterpret_cast<float4*>(cum_row + j0) = r;
              }
            } else {
              cum_row[j0] = r.x;
              if (j0 + 1 < n_keys) cum_row[j0 + 1] = r.y;
              if (j0 + 2 < n_keys) cum_row[j0 + 2] = r.z;
              if (j0 + 3 < n_keys) cum_row[j0 + 3] = r.w;
            }
            const float rv[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
            for (int k = 0; k < 4; ++k)
              if (j0 + k < n_keys) { bmax = fmaxf(bmax, rv[k]); bsum += rv[k]; }
          }
        }
        if (p.blk_bs > 0) {
          // A block of blk_bs keys is held by blk_bs / 4 consecutive lanes
          // (blocks are aligned to the chunk): reduce across that lane group.
          const int tpb = p.blk_bs >> 2;
          for (int off = 1; off < tpb; off <<= 1) {
            bmax = fmaxf(bmax, __shfl_xor(bmax, off, kWave));
            bsum += __shfl_xor(bsum, off, kWave);
          }
          const int key_b = start + (j0 / p.blk_bs) * p.blk_bs;
          // only blocks that start inside this chunk's keys (threads past the
          // chunk would otherwise name blocks of the next chunk)
          if ((tid & (tpb - 1)) == 0 && key_b < start + n_keys) {
            const size_t o = (size_t)b * p.blk_seq_stride + (size_t)kvh * p.blk_head_stride + key_b / p.blk_bs;
            if (p.blk_max) p.blk_max[o] = bmax;
            if (p.blk_mean) p.blk_mean[o] = bsum / (float)min(p.blk_bs, L - key_b);
          }
        }
      }
    } else {
      // The row did not complete in time: hand the chunk-relative values to
      // the fix-up pass, which scales them once the row's lse is known.
      if constexpr (HAS_V) {
#pragma unroll
        for (int i = 0; i < kNO; ++i) {
          const int idx = tid + i * kThreads;
          if (idx < GT * D) p.part_o[((ml_base + (size_t)(idx / D) * p.n_chunks)) * D + idx % D] = ov[i];
        }
      }
      for (int j = tid; j < n_keys; j += kThreads) {
#pragma unroll
        for (int h = 0; h < GT; ++h)
          p.raw[((size_t)b * p.num_q_heads + h0 + h) * p.raw_stride + start + j] = p_lds[j * GT + h];
      }
    }
    if (tid == 0) p.chunk_flag[row * p.n_chunks + chunk_id] = ok ? 0u : 1u;
  }
}

// ---- bf16 logits-only pass (indexer scores) ---------------------------------
// Emit raw scale * q.k for every key and up to 32 query heads of a KV head
// per workgroup: NCT 16-column B tiles of Q^T share each K tile, so the K
// stream is read once for the whole group.  No softmax, no V, no LDS tile.
// ALIGNED: every logits row is 16-byte aligned (the host checks the base and
// the stride), so whole chunks take 16-byte stores; otherwise every tile is
// written through a per-wave LDS slice as runs of 16 consecutive keys.  The
// two are separate instantiations so the aligned one keeps its own code.
template <int D, int NCT, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void decode_logits_mfma(PartialParams p) {
  constexpr int NU = D / 32;
  constexpr int QB = 4;                      // K tiles per load batch
  constexpr int GTL = 16 * NCT;
  __shared__ int page_lds[KVSEL_MAX_CHUNK / 16 + 2];
  __shared__ float lg_stage[ALIGNED ? 1 : kWaves][16 * 16];   // per wave: one tile, [head slot][key]
  const int C = p.chunk;
  const int chunk_id = blockIdx.x;
  const int kvh = blockIdx.y / p.hgroups;
  const int hg = blockIdx.y % p.hgroups;
  const int b = blockIdx.z;
  const int L = p.seq_lens[b];
  const int start = chunk_id * C;
  if (start >= L) return;
  const int n_keys = min(C, L - start);
  const int n_heads = min(GTL, p.group - hg * GTL);    // real heads in this pass
  const int h0 = kvh * p.group + hg * GTL;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int col = lane & 15, grp = lane >> 4;
  const int P = 1 << p.page_log2;
  const int first_page = start >> p.page_log2;
  const int n_pages = ((start + n_keys - 1) >> p.page_log2) - first_page + 1;
  for (int i = tid; i < n_pages; i += kThreads)
    page_lds[i] = p.block_table[(size_t)b * p.max_pages + first_page + i];
  bf16x8 qb[NCT][NU];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int hh = ct * 16 + col;
      uint4 w = make_uint4(0, 0, 0, 0);
      if (hh < n_heads) w = ld16(p.q + (((size_t)b * p.num_q_heads + h0 + hh) * D + u * 32 + grp * 8) * 2);
      qb[ct][u] = __builtin_bit_cast(bf16x8, w);
    }
  __syncthreads();
  const size_t head_stride = (size_t)P * D * 2;
  const size_t page_stride = head_stride * p.num_kv_heads;
  const int per_wave = C / kWaves;
  const int nt = per_wave / 16;
  const int wbase = wave * per_wave;
  const bool vec = ALIGNED && n_keys == C;
  for (int t0 = 0; t0 < nt; t0 += QB) {
    bf16x8 kb[QB][NU];
    auto krow = [&](int key) -> const uint8_t* {
      const int j = start + key;
      const int pg = page_lds[(j >> p.page_log2) - first_page];
      return p.k_pages + (size_t)pg * page_stride + kvh * head_stride + (size_t)(j & (P - 1)) * D * 2;
    };
#pragma unroll
    for (int t = 0; t < QB; ++t) {
      if constexpr (KVSEL_K_LINES) {
        const int key = wbase + min(t0 + t, nt - 1) * 16 + (col & 7);
        const int sg = (grp + 4 * (col >> 3)) * 16;
        const uint8_t* ra = krow(min(key, n_keys - 1)) + sg;
        const uint8_t* rb = krow(min(key + 8, n_keys - 1)) + sg;
#pragma unroll
        for (int v = 0; v < NU / 2; ++v) {
          kb[t][2 * v] = __builtin_bit_cast(bf16x8, KVSEL_NT_K_QK ? ld_kv(ra + v * 128) : ld16(ra + v * 128));
          kb[t][2 * v + 1] = __builtin_bit_cast(bf16x8, KVSEL_NT_K_QK ? ld_kv(rb + v * 128) : ld16(rb + v * 128));
        }
      } else {
        const uint8_t* rp = krow(min(wbase + min(t0 + t, nt - 1) * 16 + col, n_keys - 1)) + grp * 16;
#pragma unroll
        for (int u = 0; u < NU; ++u) kb[t][u] = __builtin_bit_cast(bf16x8, KVSEL_NT_K_QK ? ld_kv(rp + u * 64) : ld16(rp + u * 64));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < QB; ++t) {
      if (t0 + t < nt) {
        if constexpr (KVSEL_K_LINES) {
#pragma unroll
          for (int v = 0; v < NU / 2; ++v) k_line_exchange(kb[t][2 * v], kb[t][2 * v + 1], col < 8);
        }
        const int k0 = wbase + (t0 + t) * 16 + grp * 4;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int u = 0; u < NU; ++u)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[t][u], qb[ct][u], acc, 0, 0, 0);
          const int hh = ct * 16 + col;
          if constexpr (ALIGNED) {
            if (hh < n_heads) {
              float* lg = p.logits + ((size_t)b * p.num_q_heads + h0 + hh) * p.logits_stride + start;
              if (vec) {
                *reinterpret_cast<float4*>(lg + k0) =
                    make_float4(acc[0] * p.scale, acc[1] * p.scale, acc[2] * p.scale, acc[3] * p.scale);
              } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  if (k0 + i < n_keys) lg[k0 + i] = acc[i] * p.scale;
              }
            }
          } else {
            // Rows that are not 16-byte aligned: the tile passes through this
            // wave's LDS slice so that a store instruction writes runs of 16
            // consecutive keys (4 heads x 16 keys) instead of 4-key pieces of
            // 16 heads.  LDS operations of one wave complete in order; the
            // barriers keep the compiler from moving the reads above the
            // writes or the next writes above them.
            float* sl = lg_stage[wave];
#pragma unroll
            for (int i = 0; i < 4; ++i) sl[col * 16 + grp * 4 + i] = acc[i] * p.scale;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const int key = wbase + (t0 + t) * 16 + col;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int hl = r * 4 + grp;
              if (ct * 16 + hl < n_heads && key < n_keys)
                p.logits[((size_t)b * p.num_q_heads + h0 + ct * 16 + hl) * p.logits_stride + start + key] =
                    sl[hl * 16 + col];
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
          }
        }
      }
    }
  }
}

template <int D, int NCT>
void launch_logits(bool aligned, dim3 grid, hipStream_t stream, const PartialParams& pp) {
  if (aligned) hipLaunchKernelGGL((decode_logits_mfma<D, NCT, true>), grid, dim3(kThreads), 0, stream, pp);
  else hipLaunchKernelGGL((decode_logits_mfma<D, NCT, false>), grid, dim3(kThreads), 0, stream, pp);
}

// ---- combine ----------------------------------------------------------------
// One workgroup per (sequence, query head): global max M over the chunk
// partials, weights w_c = exp(m_c - M), l = sum w_c l_c, out = sum w_c o_c / l,
// lse = M + ln l.  The chunk rows of o are summed by 8 thread groups in
// parallel (float4 per thread), then across the groups in LDS.
struct CombineParams {
  const int32_t* seq_lens;
  const float* part_o;
  const float2* part_ml;
  float* out;       // [B][Hq][D] or null
  float* lse;       // [B][Hq] or null
  float* lse_ws;    // [B][Hq]
  int num_q_heads, chunk, n_chunks, D;
  // Fix-up of chunks the in-kernel normalisation left behind (null: none).
  const uint32_t* chunk_flag;  // [B][H_kv][n_chunks]
  int group, num_kv_heads;
  float* probs;                // [B][Hq][probs_stride] or null
  int64_t probs_stride;
  const float* raw;            // chunk-relative exp values of flagged chunks
  int64_t raw_stride;
  float* cum;                  // [B][H_kv][cum_stride] or null
  int64_t cum_stride;
  float decay;
  // The pass's posts of this (sequence, query head), [n_chunks][2] words,
  // or null.  The combine zeroes those of the row's chunks: a zero pair never
  // validates, so a later execution with the same tag (a replayed graph)
  // cannot accept a post left by an earlier one.
  unsigned long long* lse_post;
  int blk_bs;                  // > 0: block aggregates of the chunks finished here
  float* blk_max;
  float* blk_mean;
  int64_t blk_head_stride, blk_seq_stride;
  // 1: chunks that completed in the pass hold exp(m_chunk - lse) o_chunk
  // (flag 0), the others the plain partial output (flag 1); the row's first
  // chunk wrote lse when it completed.
  int prescaled;
};

constexpr int kCombThreads = 256;
constexpr int kCombPre = 4;    // partial-output rows per thread loaded up front

__device__ __forceinline__ float block_reduce(float v, float* scratch, bool is_max) {
  v = is_max ? wave_max(v) : wave_sum(v);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  float r = scratch[0];
#pragma unroll
  for (int w = 1; w < kCombThreads / kWave; ++w) r = is_max ? fmaxf(r, scratch[w]) : r + scratch[w];
  return r;
}

template <bool HAS_V>
__global__ __launch_bounds__(kCombThreads) void decode_combine(CombineParams p) {
  extern __shared__ float csm[];
  float* w_lds = csm;                          // [n_chunks]
  float* red = csm + p.n_chunks;               // [kCombThreads][4]: one float4 per thread
  float* scratch = red + 4 * kCombThreads;     // [kCombThreads / kWave]
  const int bh = blockIdx.x;
  const int b = bh / p.num_q_heads;
  const int L = p.seq_lens[b];
  const float2* ml = p.part_ml + (size_t)bh * p.n_chunks;
  const int tid = threadIdx.x;
  // Every global load of the common case is issued before the first
  // reduction, and before the row's chunk count (from seq_lens) is known:
  // the chunk (max, sum) pairs, the first kCombPre partial outputs of this
  // thread's chunk group and the fix-up flags are read for every workspace
  // slot, and the slots past the row's chunks are masked afterwards.
  const bool do_out = HAS_V && p.out != nullptr;
  const int D4 = p.D / 4;
  const int d4 = tid % D4, cg = tid / D4, ng = kCombThreads / D4;
  const float4* po = reinterpret_cast<const float4*>(p.part_o + (size_t)bh * p.n_chunks * p.D);
  float2 mv = make_float2(kNegInf, 0.f);
  if (tid < p.n_chunks) mv = ml[tid];
  float4 pre[kCombPre];
#pragma unroll
  for (int i = 0; i < kCombPre; ++i) {
    const int c = cg + i * ng;
    pre[i] = (do_out && c < p.n_chunks) ? po[(size_t)c * D4 + d4] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const bool pres = HAS_V && p.prescaled != 0;
  const size_t row = (size_t)b * p.num_kv_heads + (bh % p.num_q_heads) / p.group;
  const uint32_t* flags = p.chunk_flag != nullptr ? p.chunk_flag + row * p.n_chunks : nullptr;
  const bool fix_head = flags != nullptr && (bh % p.num_q_heads) % p.group == 0;
  const bool read_flags = fix_head || (pres && flags);
  const uint32_t f0 = read_flags && tid < p.n_chunks ? flags[tid] : 0u;
  const int nc = (L + p.chunk - 1) / p.chunk;
  if (tid >= nc) mv = make_float2(kNegInf, 0.f);
#pragma unroll
  for (int i = 0; i < kCombPre; ++i)
    if (cg + i * ng >= nc) pre[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (p.lse_post) {
    // The pass that wrote these posts has completed (stream order), so no
    // reader is left; zero the pairs of every chunk the pass had.
    unsigned long long* pw = p.lse_post + 2 * (size_t)bh * p.n_chunks;
    for (int i = tid; i < 2 * nc; i += kCombThreads) pw[i] = 0ull;
  }
  int any = tid < nc ? (int)f0 : 0;
  if (read_flags)
    for (int c = tid + kCombThreads; c < nc; c += kCombThreads) any |= (int)flags[c];

  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  auto add = [&](float w, const float4& v) {
    o.x = fmaf(w, v.x, o.x); o.y = fmaf(w, v.y, o.y);
    o.z = fmaf(w, v.z, o.z); o.w = fmaf(w, v.w, o.w);
  };
  // Cross-group sum of o and the store of out (divided by den).
  auto finish_out = [&](float den) {
    reinterpret_cast<float4*>(red)[cg * D4 + d4] = o;
    __syncthreads();
    if (tid < p.D) {
      float r = 0.f;
      for (int g = 0; g < ng; ++g) r += red[g * p.D + tid];
      p.out[(size_t)bh * p.D + tid] = r / den;
    }
  };
  if (pres && !__syncthreads_or(any)) {
    // Every chunk of the row completed in the pass: out is the plain sum of
    // the weighted partial outputs, and lse is already written.
#pragma unroll
    for (int i = 0; i < kCombPre; ++i)
      if (cg + i * ng < nc) add(1.f, pre[i]);
    for (int c = cg + kCombPre * ng; c < nc; c += ng) add(1.f, po[(size_t)c * D4 + d4]);
    finish_out(1.f);
    return;
  }

  float M = mv.x;
  for (int c = tid + kCombThreads; c < nc; c += kCombThreads) M = fmaxf(M, ml[c].x);
  M = block_reduce(M, scratch, true);
  const float Ms = M * kLog2e;
  float l = 0.f;
  for (int c = tid; c < nc; c += kCombThreads) {
    const float2 v = c == tid ? mv : ml[c];
    const float w = exp2_hw(fmaf(v.x, kLog2e, -Ms));
    w_lds[c] = w;
    l = fmaf(w, v.y, l);
  }
  l = block_reduce(l, scratch, false);   // also orders the w_lds writes
  if (pres) {
    // Mixed row: weighted chunks count once, plain ones get exp(m_c - lse).
    const float lse2 = M * kLog2e + log2_hw(l);
    for (int c = tid; c < nc; c += kCombThreads)
      w_lds[c] = flags[c] ? exp2_hw(fmaf(ml[c].x, kLog2e, -lse2)) : 1.f;
    __syncthreads();
  }
  if (do_out) {
#pragma unroll
    for (int i = 0; i < kCombPre; ++i) {
      const int c = cg + i * ng;
      if (c < nc) add(w_lds[c], pre[i]);
    }
    for (int c = cg + kCombPre * ng; c < nc; c += ng) add(w_lds[c], po[(size_t)c * D4 + d4]);
    finish_out(pres ? 1.f : l);
  }
  if (tid == 0) {
    const float v = M + log2_hw(l) * kLn2;
    p.lse_ws[bh] = v;
    if (p.lse) p.lse[bh] = v;
  }
  if (!fix_head) return;
  // The first head of each group finishes its row's flagged chunks: raw
  // holds exp(s - m_chunk) for every head of the group; scale by
  // exp(m_chunk - lse), write the probabilities and fold cum.
  const int G = p.group;
  if (!__syncthreads_or(any)) return;
  __shared__ float lse_g[8];
  for (int g = 0; g < G; ++g) {
    const float2* mlg = p.part_ml + (size_t)(bh + g) * p.n_chunks;
    float Mg = kNegInf;
    for (int c = tid; c < nc; c += kCombThreads) Mg = fmaxf(Mg, mlg[c].x);
    Mg = block_reduce(Mg, scratch, true);
    float lg = 0.f;
    for (int c = tid; c < nc; c += kCombThreads) lg = fmaf(mlg[c].y, exp2_hw((mlg[c].x - Mg) * kLog2e), lg);
    lg = block_reduce(lg, scratch, false);
    if (tid == 0) lse_g[g] = Mg + log2_hw(lg) * kLn2;
  }
  __syncthreads();
  for (int c = 0; c < nc; ++c) {
    if (flags[c] == 0) continue;
    const int start = c * p.chunk;
    const int n_keys = min(p.chunk, L - start);
    for (int j = tid; j < n_keys; j += kCombThreads) {
      float acc = 0.f;
      for (int g = 0; g < G; ++g) {
        const size_t bhg = (size_t)bh + g;
        const float f = exp2_hw((p.part_ml[bhg * p.n_chunks + c].x - lse_g[g]) * kLog2e);
        const float pv = p.raw[bhg * p.raw_stride + start + j] * f;
        if (p.probs) p.probs[bhg * p.probs_stride + start + j] = pv;
        acc += pv;
      }
      if (p.cum) {
        float* cp = p.cum + row * p.cum_stride + start + j;
        *cp = fmaf(p.decay, *cp, acc);
      }
    }
    if (p.blk_bs > 0) {
      __syncthreads();                     // this chunk's cum writes are visible to the block
      const float* cr = p.cum + row * p.cum_stride;
      const int kvh = (int)(row % p.num_kv_heads);
      for (int bl = tid; bl * p.blk_bs < n_keys; bl += kCombThreads) {
        const int k0 = start + bl * p.blk_bs, k1 = min(k0 + p.blk_bs, L);
        float mx = kNegInf, sm = 0.f;
        for (int k = k0; k < k1; ++k) { mx = fmaxf(mx, cr[k]); sm += cr[k]; }
        const size_t o = (size_t)b * p.blk_seq_stride + (size_t)kvh * p.blk_head_stride + k0 / p.blk_bs;
        if (p.blk_max) p.blk_max[o] = mx;
        if (p.blk_mean) p.blk_mean[o] = sm / (float)(k1 - k0);
      }
    }
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

// VEC: 4 consecutive keys per thread with 16-byte accesses (every stride a
// multiple of 4 and every base 16-byte aligned).
template <bool VEC>
__global__ __launch_bounds__(kFinThreads) void decode_finalize(FinalizeParams p) {
  const int b = blockIdx.z;
  const int c = blockIdx.y;
  const int L = p.seq_lens[b];
  const int start = blockIdx.x * p.keys_per_block;
  if (start >= L) return;
  const int end = min(L, start + p.keys_per_block);
  const int h0 = c * p.group;
  const size_t bh0 = (size_t)b * p.num_q_heads + h0;
  float* cp = p.cum ? p.cum + ((size_t)b * p.num_kv_heads + c) * p.cum_stride : nullptr;
  if constexpr (VEC) {
    for (int j = start + threadIdx.x * 4; j < end; j += kFinThreads * 4) {
      if (j + 3 < end) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int g = 0; g < p.group; ++g) {
          const float ls = p.lse_ws[bh0 + g] * kLog2e;
          const float4 s = *reinterpret_cast<const float4*>(p.logits + (bh0 + g) * p.logits_stride + j);
          float4 e;
          e.x = exp2_hw(fmaf(s.x, kLog2e, -ls)); e.y = exp2_hw(fmaf(s.y, kLog2e, -ls));
          e.z = exp2_hw(fmaf(s.z, kLog2e, -ls)); e.w = exp2_hw(fmaf(s.w, kLog2e, -ls));
          if (p.probs) {
#if KVSEL_NT_PROBS
            st16_stream(p.probs + (bh0 + g) * p.probs_stride + j, e);
#else
            *reinterpret_cast<float4*>(p.probs + (bh0 + g) * p.probs_stride + j) = e;
#endif
          }
          acc.x += e.x; acc.y += e.y; acc.z += e.z; acc.w += e.w;
        }
        if (cp) {
          float4 cv = *reinterpret_cast<float4*>(cp + j);
          cv.x = fmaf(p.decay, cv.x, acc.x); cv.y = fmaf(p.decay, cv.y, acc.y);
          cv.z = fmaf(p.decay, cv.z, acc.z); cv.w = fmaf(p.decay, cv.w, acc.w);
          *reinterpret_cast<float4*>(cp + j) = cv;
        }
      } else {
        for (int jj = j; jj < end; ++jj) {
          float acc = 0.f;
          for (int g = 0; g < p.group; ++g) {
            const float ls = p.lse_ws[bh0 + g] * kLog2e;
            const float e = exp2_hw(fmaf(p.logits[(bh0 + g) * p.logits_stride + jj], kLog2e, -ls));
            if (p.probs) p.probs[(bh0 + g) * p.probs_stride + jj] = e;
            acc += e;
          }
          if (cp) cp[jj] = fmaf(p.decay, cp[jj], acc);
        }
      }
    }
  } else {
    for (int j = start + threadIdx.x; j < end; j += kFinThreads) {
      float acc = 0.f;
      for (int g = 0; g < p.group; ++g) {
        const float ls = p.lse_ws[bh0 + g] * kLog2e;
        const float e = exp2_hw(fmaf(p.logits[(bh0 + g) * p.logits_stride + j], kLog2e, -ls));
        if (p.probs) p.probs[(bh0 + g) * p.probs_stride + j] = e;
        acc += e;
      }
      if (cp) cp[j] = fmaf(p.decay, cp[j], acc);
    }
  }
}

template <bool BF16, int D, int GT, bool HAS_V, bool WL>
hipError_t launch_partial_t(const PartialParams& pp, dim3 grid, size_t lds, hipStream_t s) {
  if constexpr (BF16)
    hipLaunchKernelGGL((decode_partial_mfma<D, GT, HAS_V, WL, false>), grid, dim3(kThreads), lds, s, pp);
  else
    hipLaunchKernelGGL((decode_partial<false, D, GT, HAS_V, WL>), grid, dim3(kThreads), lds, s, pp);
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

template <int D>
hipError_t launch_coop_d(const PartialParams& pp, int gt, bool has_v, dim3 grid, size_t lds, hipStream_t s) {
#define KVSEL_COOP(G)                                                                                        \
  if (has_v)                                                                                                 \
    hipLaunchKernelGGL((decode_partial_mfma<D, G, true, false, true>), grid, dim3(kThreads), lds, s, pp);   \
  else                                                                                                       \
    hipLaunchKernelGGL((decode_partial_mfma<D, G, false, false, true>), grid, dim3(kThreads), lds, s, pp);  \
  break;
  switch (gt) {
    case 1: KVSEL_COOP(1)
    case 2: KVSEL_COOP(2)
    case 4: KVSEL_COOP(4)
    case 8: KVSEL_COOP(8)
    default: return hipErrorInvalidValue;
  }
#undef KVSEL_COOP
  return hipGetLastError();
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

DecodePlan plan_decode(int num_seqs, int num_kv_heads, int num_q_heads, int head_dim,
                       int max_seq_len, bool need_scratch) {
  DecodePlan pl{};
  const int G = num_q_heads / num_kv_heads;
  pl.gt = G >= 8 ? 8 : G;
  pl.hgroups = G / pl.gt;
  // Largest chunk (<= KVSEL_MAX_CHUNK keys) that still gives the grid
  // >= KVSEL_MIN_WGS workgroups, never below 64 keys.
  int chunk = KVSEL_FIXED_CHUNK > 0 ? KVSEL_FIXED_CHUNK : KVSEL_MAX_CHUNK;
  while (KVSEL_FIXED_CHUNK == 0 && chunk > 64) {
    const long long wgs = (long long)num_seqs * num_kv_heads * pl.hgroups *
                          ((max_seq_len + chunk - 1) / chunk);
    if (wgs >= KVSEL_MIN_WGS) break;
    chunk /= 2;
  }
  pl.chunk = chunk;
  pl.n_chunks = (max_seq_len + chunk - 1) / chunk;
  const size_t bh = (size_t)num_seqs * num_q_heads;
  pl.part_o_bytes = align256(bh * pl.n_chunks * head_dim * sizeof(float));
  pl.part_ml_bytes = align256(bh * pl.n_chunks * sizeof(float2));
  pl.lse_bytes = align256(bh * sizeof(float));
  pl.scratch_bytes = need_scratch ? align256(bh * (size_t)max_seq_len * sizeof(float)) : 0;
  const size_t rows = (size_t)num_seqs * num_kv_heads;
  pl.sync_bytes = align256(bh * pl.n_chunks * 2 * sizeof(unsigned long long)) +
                  align256(rows * pl.n_chunks * sizeof(uint32_t));
  pl.total_bytes = pl.part_o_bytes + pl.part_ml_bytes + pl.lse_bytes + pl.scratch_bytes + pl.sync_bytes;
  return pl;
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& pl, hipStream_t stream) {
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  float* part_o = reinterpret_cast<float*>(ws);
  float2* part_ml = reinterpret_cast<float2*>(ws + pl.part_o_bytes);
  float* lse_ws = reinterpret_cast<float*>(ws + pl.part_o_bytes + pl.part_ml_bytes);
  float* scratch = reinterpret_cast<float*>(ws + pl.part_o_bytes + pl.part_ml_bytes + pl.lse_bytes);
  uint8_t* sync_base = ws + pl.part_o_bytes + pl.part_ml_bytes + pl.lse_bytes + pl.scratch_bytes;
  const size_t rows = (size_t)a.num_seqs * a.num_kv_heads;

  const bool use_v = a.v_pages != nullptr && a.out != nullptr;
  const bool need_norm = !a.emit_logits && (a.probs != nullptr || a.cum != nullptr);
  // In-kernel normalisation: bf16, one workgroup serves a whole group.
  // The lse of a row's chunks are gathered in LDS ([GT][n_chunks] floats in
  // the area of the P.V reduction tile), hence a bound on the chunk count
  // (kWaves * d: 16 KB at G = 8 and d = 128).
  const bool coop = KVSEL_COOP_NORM && a.bf16 && need_norm && pl.hgroups == 1 &&
                    pl.n_chunks <= kWaves * a.head_dim && (a.probs != nullptr || pl.scratch_bytes > 0);
  float* logits = nullptr;
  int64_t logits_stride = 0;
  if (!coop) {
    if (a.probs) {
      logits = a.probs;
      logits_stride = a.probs_stride;
    } else if (need_norm) {
      logits = scratch;
      logits_stride = a.max_seq_len;
    }
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
  pp.num_rows = (int)rows;
  const size_t post_bytes = align256((size_t)a.num_seqs * a.num_q_heads * pl.n_chunks * 2 * sizeof(unsigned long long));
  pp.lse_post = reinterpret_cast<unsigned long long*>(sync_base);
  pp.chunk_flag = reinterpret_cast<uint32_t*>(sync_base + post_bytes);
  pp.epoch = a.epoch;
  pp.wait_ticks = a.wait_ticks;
  pp.probs = a.probs;
  pp.probs_stride = a.probs_stride;
  pp.raw = a.probs ? a.probs : scratch;
  pp.raw_stride = a.probs ? a.probs_stride : a.max_seq_len;
  pp.cum = a.cum;
  pp.cum_stride = a.cum_stride;
  pp.decay = a.decay;
  // Block aggregates inside the normalising pass when the blocks tile its
  // chunks (power-of-two sizes 4..256 dividing the chunk); otherwise by the
  // aggregation kernel after the pass.
  const bool blk = a.blk_bs > 0 && (a.blk_max || a.blk_mean);
  const bool blk_fused = blk && coop && (a.blk_bs & (a.blk_bs - 1)) == 0 && a.blk_bs >= 4 &&
                         a.blk_bs <= 256 && pl.chunk % a.blk_bs == 0;
  if (coop && use_v) pp.lse_out = a.lse;
  if (blk_fused) {
    pp.blk_bs = a.blk_bs;
    pp.blk_max = a.blk_max;
    pp.blk_mean = a.blk_mean;
    pp.blk_head_stride = a.blk_head_stride;
    pp.blk_seq_stride = a.blk_seq_stride;
  }

  // Pure logits (indexer scores): the dedicated kernel serving up to 32 heads
  // per K read.
  if (a.bf16 && a.emit_logits && !a.out && !a.lse && !a.cum && a.probs) {
    const int G = a.num_q_heads / a.num_kv_heads;
    const int nct = G > 16 ? 2 : 1;
    pp.hgroups = (G + 16 * nct - 1) / (16 * nct);
    // its own chunk: the largest (<= the plan's) that gives this grid
    // KVSEL_MIN_WGS workgroups, never below 128 keys
    int lchunk = pl.chunk;
    while (lchunk > 128 && (long long)a.num_seqs * a.num_kv_heads * pp.hgroups *
                                   ((a.max_seq_len + lchunk - 1) / lchunk) < KVSEL_MIN_WGS)
      lchunk /= 2;
    pp.chunk = lchunk;
    pp.n_chunks = (a.max_seq_len + lchunk - 1) / lchunk;
    const dim3 lgrid(pp.n_chunks, a.num_kv_heads * pp.hgroups, a.num_seqs);
    const bool al = (pp.logits_stride & 3) == 0 && (reinterpret_cast<uintptr_t>(pp.logits) & 15) == 0;
    if (a.head_dim == 128) {
      if (nct == 2) launch_logits<128, 2>(al, lgrid, stream, pp);
      else launch_logits<128, 1>(al, lgrid, stream, pp);
    } else {
      if (nct == 2) launch_logits<64, 2>(al, lgrid, stream, pp);
      else launch_logits<64, 1>(al, lgrid, stream, pp);
    }
    return hipGetLastError();
  }
  const dim3 grid(pl.n_chunks, a.num_kv_heads * pl.hgroups, a.num_seqs);
  // the bf16 pass sums its waves through one [GT][D] tile, which the
  // in-kernel normalisation then reuses for the row's [GT][n_chunks] posts
  const size_t red_floats = !a.bf16 ? (size_t)kWaves * pl.gt * a.head_dim
                                    : (size_t)pl.gt * (coop ? std::max(a.head_dim, pl.n_chunks) : a.head_dim);
  const size_t lds = (size_t)pl.gt * pl.chunk * sizeof(float) + red_floats * sizeof(float) +
                     (a.bf16 ? 2 * kWaves * 16 * sizeof(float) : 0) + pl.gt * sizeof(float2) +
                     ((size_t)pl.chunk / 16 + 2) * sizeof(int);
  const bool wl = logits != nullptr;
  hipError_t e;
  if (coop) {
    const dim3 cgrid((unsigned)(rows * (size_t)pl.n_chunks));
    e = a.head_dim == 128 ? launch_coop_d<128>(pp, pl.gt, use_v, cgrid, lds, stream)
                          : launch_coop_d<64>(pp, pl.gt, use_v, cgrid, lds, stream);
  } else if (a.bf16) {
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
      cp.group = pp.group;
      cp.num_kv_heads = a.num_kv_heads;
      if (coop) {
        cp.blk_bs = pp.blk_bs;
        cp.blk_max = pp.blk_max;
        cp.blk_mean = pp.blk_mean;
        cp.blk_head_stride = pp.blk_head_stride;
        cp.blk_seq_stride = pp.blk_seq_stride;
        cp.chunk_flag = pp.chunk_flag;
        cp.lse_post = pp.lse_post;
        cp.probs = a.probs;
        cp.probs_stride = a.probs_stride;
        cp.raw = pp.raw;
        cp.raw_stride = pp.raw_stride;
        cp.cum = a.cum;
        cp.cum_stride = a.cum_stride;
        cp.decay = a.decay;
        cp.prescaled = use_v ? 1 : 0;
      }
      const dim3 cgrid(a.num_seqs * a.num_q_heads);
      const size_t clds = ((size_t)pl.n_chunks + 4 * kCombThreads + 8) * sizeof(float);
      if (use_v)
        hipLaunchKernelGGL(decode_combine<true>, cgrid, dim3(kCombThreads), clds, stream, cp);
      else
        hipLaunchKernelGGL(decode_combine<false>, cgrid, dim3(kCombThreads), clds, stream, cp);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }

  auto blocks_after = [&]() -> hipError_t {
    if (!blk || blk_fused) return hipSuccess;
    return launch_block_aggregate(a.cum, a.cum_stride, a.seq_lens, a.num_seqs, a.num_kv_heads, a.max_seq_len,
                                  a.blk_bs, false, false, a.blk_max, a.blk_mean, a.blk_head_stride,
                                  a.blk_seq_stride, stream);
  };
  if (coop) return blocks_after();   // the combine finished any chunk left behind
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
    auto al16 = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; };
    const bool vec = logits_stride % 4 == 0 && al16(logits) &&
                     (!a.probs || (a.probs_stride % 4 == 0 && al16(a.probs))) &&
                     (!a.cum || (a.cum_stride % 4 == 0 && al16(a.cum)));
    if (vec)
      hipLaunchKernelGGL(decode_finalize<true>, fgrid, dim3(kFinThreads), 0, stream, fp);
    else
      hipLaunchKernelGGL(decode_finalize<false>, fgrid, dim3(kFinThreads), 0, stream, fp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return blocks_after();
}

}  // namespace kvsel
