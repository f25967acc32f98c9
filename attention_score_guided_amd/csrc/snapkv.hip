// SnapKV observation-window vote ([EVICT] "KV-cache eviction strategies",
// §4.3): the last W prompt queries (the observation window) take a causal
// softmax over the prompt's keys; each prefix key's vote is the sum of the
// probabilities it receives from the window queries of a head, optionally
// summed over the query heads of a KV group; the vote is then max-pooled
// (stride 1, same length) so the neighbours of a heavy position survive.
//
// The window logits are a real dense contraction: for one query head, the
// W x d window queries against every key, 16 keys x 16 window rows per
// v_mfma_f32_16x16x32_bf16 chain.  A workgroup serves all G query heads of
// a KV head for a run of chunks of one sequence: each 128-key chunk is
// staged in LDS once and read by every wave as MFMA fragments.  The pass is
// bound by latency (dependent MFMA -> FMA -> exp -> add chains), so the
// design favours occupancy: 128-key chunks (~37 KB of LDS), two tiles in
// flight and no register prefetch of the next chunk keep a workgroup within
// 128 VGPRs, and four workgroups per CU (four waves per SIMD) overlap one
// workgroup's chunk loads with the others' compute.  The per-logit vector
// work is one FMA, one exp2 (quarter rate) and one add on tiles that need no
// causal mask.  Two passes over K:
//   pass 1  per window row, (max, sum of exp) over the workgroup's keys, in
//           base-2 units with a lazily moved reference (the running sum is
//           rescaled only when a logit exceeds the reference by 2^64);
//   combine per window row: lse over the workgroups' partials;
//   pass 2  recompute the logits of each chunk plus a halo of the pool
//           radius on each side with the window rows as the MFMA A operand, so a lane holds
//           four rows of one key: p = exp2(s - lse2), column sums by local
//           adds and two cross-lane steps, the group sum in head order, the
//           max-pool, and the final votes of the chunk's prefix keys.
// Every output element has one writer; there are no atomics.
#include <algorithm>
#include <type_traits>

#include "device_common.hpp"
#include "kvsel_internal.hpp"

namespace kvsel {

namespace {


constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
#ifndef KVSEL_VOTE_STAGE
#define KVSEL_VOTE_STAGE 128  // keys staged per chunk (8 tiles)
#endif
constexpr int kStage = KVSEL_VOTE_STAGE;
constexpr int kTiles = kStage / 16;
constexpr int kMaxHalo = 8;             // pass 2: extra keys on each side = the pool radius (<= 8)
#ifndef KVSEL_VOTE_WGS
#define KVSEL_VOTE_WGS 1024   // grid target (128K case: ~1000 workgroups, one round of 4 per CU)
#endif
#ifndef KVSEL_VOTE_TN1
#define KVSEL_VOTE_TN1 2     // pass 1: fully visible tiles computed together
#endif
#ifndef KVSEL_VOTE_TN2
#define KVSEL_VOTE_TN2 2     // pass 2: fully visible tiles computed together (2 or 4)
#endif
#ifndef KVSEL_VOTE_WPE1
#define KVSEL_VOTE_WPE1 4    // >0: occupancy hint (waves per SIMD) for pass 1
#endif
#ifndef KVSEL_VOTE_WPE2
#define KVSEL_VOTE_WPE2 4    // >0: occupancy hint (waves per SIMD) for pass 2
#endif
constexpr int kMaxWgs = KVSEL_VOTE_WGS;  // grid target: chunks are grouped into runs beyond it
constexpr float kRescale = 64.f;        // pass 1: move the reference past this (base-2 units)

struct VoteParams {
  const uint8_t* k_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint8_t* q_win;   // [B][Hq][W][D] bf16
  int num_kv_heads, num_q_heads, window, page_log2, max_pages, radius;
  int cpw1, n_run1;       // pass 1: chunks per workgroup, runs per sequence
  int cpw2;               // pass 2: chunks per workgroup
  int halo, outc;         // pass 2: extra keys on each side (the pool radius), keys voted per chunk
  bool group_sum;
  float c2;               // scale * log2(e)
  float2* part_ml;        // [B][Hq][n_run1][W]  (reference, sum) in base-2 units
  const float* lse2;      // [B][Hq][W]          row lse in base-2 units
  float* votes;           // [B][H_out][votes_stride]
  int64_t votes_stride;
};

// Window rows of head h as MFMA fragments: lane (row = rt*16 + lane%16,
// dims u*32 + (lane/16)*8 .. +8).  Rows past the window are zero.
template <int D, int RT>
__device__ __forceinline__ void load_q(const VoteParams& p, int b, int h, int col, int grp,
                                       bf16x8 (&qf)[RT][D / 32]) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rt * 16 + col;
#pragma unroll
    for (int u = 0; u < D / 32; ++u) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (row < p.window)
        w = ld16(p.q_win + ((((size_t)b * p.num_q_heads + h) * p.window + row) * D + u * 32 + grp * 8) * 2);
      qf[rt][u] = __builtin_bit_cast(bf16x8, w);
    }
  }
}

// A chunk of kStage keys in LDS, rows unpadded: 16-byte piece c of row r is
// stored at piece c ^ (r mod pieces-per-row), so the 16 rows of a fragment
// read, and the 16 pieces of a row's store, fall in distinct bank groups (no
// bank conflicts by the counters; the earlier 16-byte row padding lost 38% of
// pass 1's LDS cycles to conflicts, at the same vote time).
template <int D>
struct Stage {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kPieces = D / 8;                                   // 16-byte pieces per key
  static constexpr int kPer = (kStage * kPieces + kThreads - 1) / kThreads;  // pieces per thread
};

// Page ids of keys [k_lo, k_hi] (clamped into [0, L)) of a workgroup's run,
// read once into LDS so each chunk's key loads are a single round trip.
__device__ __forceinline__ int load_pages(const VoteParams& p, int b, int L, int k_lo, int k_hi, int* page_lds) {
  const int lo = max(k_lo, 0) >> p.page_log2;
  const int hi = min(k_hi, L - 1) >> p.page_log2;
  for (int i = threadIdx.x; i <= hi - lo; i += kThreads)
    page_lds[i] = p.block_table[(size_t)b * p.max_pages + lo + i];
  return lo;
}

// Global loads of keys kbase .. kbase + kStage - 1 (clamped into [0, L)) into
// registers, through the run's page ids in LDS (first page `pg0`).
template <int D>
__device__ __forceinline__ void stage_load(const VoteParams& p, const int* page_lds, int pg0, int kvh, int L,
                                           int kbase, uint4 (&buf)[Stage<D>::kPer]) {
  constexpr int PC = Stage<D>::kPieces;
  const int P = 1 << p.page_log2;
  const size_t head_stride = (size_t)P * D * 2;
  const size_t page_stride = head_stride * p.num_kv_heads;
#pragma unroll
  for (int r = 0; r < Stage<D>::kPer; ++r) {
    const int pi = threadIdx.x + r * kThreads;
    const int kl = min(pi / PC, kStage - 1), seg = pi % PC;
    const int key = min(max(kbase + kl, 0), L - 1);
    const int pg = page_lds[(key >> p.page_log2) - pg0];
    buf[r] = ld16_stream(p.k_pages + (size_t)pg * page_stride + kvh * head_stride +
                         (size_t)(key & (P - 1)) * D * 2 + seg * 16);
  }
}

template <int D>
__device__ __forceinline__ void stage_store(const uint4 (&buf)[Stage<D>::kPer], uint8_t* kst) {
  constexpr int PC = Stage<D>::kPieces;
#pragma unroll
  for (int r = 0; r < Stage<D>::kPer; ++r) {
    const int pi = threadIdx.x + r * kThreads;
    if (pi < kStage * PC)
      *reinterpret_cast<uint4*>(kst + (pi / PC) * Stage<D>::kRowBytes + (((pi % PC) ^ ((pi / PC) & (PC - 1))) * 16)) = buf[r];
  }
}

// Fragments of staged tile t: lane (key = t*16 + lane%16, dims u*32 +
// (lane/16)*8 .. +8).  The same registers serve as MFMA A (keys as rows) or
// B (keys as columns).
template <int D>
__device__ __forceinline__ void tile_frag(const uint8_t* kst, int t, int col, int grp, bf16x8 (&kf)[D / 32]) {
  constexpr int PC = Stage<D>::kPieces;
  const int row = t * 16 + col;
  const uint8_t* rp = kst + row * Stage<D>::kRowBytes;
#pragma unroll
  for (int u = 0; u < D / 32; ++u)
    kf[u] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(rp + (((grp + 4 * u) ^ (row & (PC - 1))) * 16)));
}

// Items of a chunk: G x kTiles (head, tile) pairs cut into kWaves contiguous
// runs, so a wave changes head (and reloads its window rows) rarely.
__device__ __forceinline__ void wave_items(int G, int wave, int& i0, int& i1) {
  const int items = G * kTiles;
  const int per = (items + kWaves - 1) / kWaves;
  i0 = wave * per;
  i1 = min(items, i0 + per);
}

// Sum of a lane's value over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four
// row-quads of one MFMA output column), with the cross-row swaps of gfx950
// (v_permlane16_swap / v_permlane32_swap: two VALU operations, no LDS
// round trip).  With the same register as both operands, the swap's two
// results hold the values of the two rows (halves) paired by it, so their sum
// is the pairwise sum in every lane.
__device__ __forceinline__ float quad_rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2) {
  const float mn = fmaxf(m, m2);
  if (mn == kNegInf) return;  // both empty
  l = l * exp2_hw(m - mn) + l2 * exp2_hw(m2 - mn);
  m = mn;
}

// Pass 1: per (run of chunks, sequence, KV head), (reference, sum of exp2)
// of every window row of every head of the group over the run's keys.
// MFMA with keys as A rows: lane (row = rt*16 + lane%16) holds keys
// key0 + (lane/16)*4 + i, i < 4.
//
// NHW > 0: the window rows of the wave's (at most NHW) heads are loaded once,
// before the chunk loop, and held in registers, so the only global loads in
// the loop are the chunk's keys.  NHW == 0: the rows are reloaded per chunk
// and head (wide groups).
template <int D, int RT, int NHW>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(KVSEL_VOTE_WPE1 > 0 ? KVSEL_VOTE_WPE1 : 1)))
void snapkv_pass1(VoteParams p) {
  constexpr int NU = D / 32;
  constexpr bool PRE = NHW > 0;
  constexpr int NS = PRE ? NHW : 1;      // register slots of window rows
  extern __shared__ __align__(16) uint8_t sm1[];
  uint8_t* kst = sm1;                                                     // [kStage][row bytes]
  float2* wml = reinterpret_cast<float2*>(sm1 + kStage * Stage<D>::kRowBytes);  // [G][kWaves][RT*16]
  int* page_lds = reinterpret_cast<int*>(wml + (p.num_q_heads / p.num_kv_heads) * kWaves * RT * 16);
  const int G = p.num_q_heads / p.num_kv_heads;
  const int run = blockIdx.x;
  const int b = blockIdx.y / p.num_kv_heads, kvh = blockIdx.y % p.num_kv_heads;
  const int L = p.seq_lens[b];
  const int c_first = run * p.cpw1;
  const int c_end = min(c_first + p.cpw1, (L + kStage - 1) / kStage);
  if (c_first >= c_end) return;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int col = lane & 15, grp = lane >> 4;
  const int prefix = L - p.window;
  for (int i = tid; i < G * kWaves * RT * 16; i += kThreads) wml[i] = make_float2(kNegInf, 0.f);
  int i0, i1;
  wave_items(G, wave, i0, i1);
  const int g_lo = i0 / kTiles;
  const int g_hi = i0 < i1 ? (i1 - 1) / kTiles : g_lo - 1;

  bf16x8 qf[NS][RT][NU];
  float m_ref[NS][RT], l_sum[NS][RT];
#pragma unroll
  for (int hs = 0; hs < NS; ++hs) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) { m_ref[hs][rt] = kNegInf; l_sum[hs][rt] = 0.f; }
    if (PRE && g_lo + hs <= g_hi) load_q<D, RT>(p, b, kvh * G + g_lo + hs, col, grp, qf[hs]);
  }
  // Merge a lane's (reference, sum) of head g into the wave's LDS slot.
  auto flush = [&](int g, float (&m_)[RT], float (&l_)[RT]) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float m = m_[rt], l = l_[rt];
      for (int off = 16; off < kWave; off *= 2) merge_ml(m, l, __shfl_xor(m, off, kWave), __shfl_xor(l, off, kWave));
      if (grp == 0) {
        float2& slot = wml[(g * kWaves + wave) * RT * 16 + rt * 16 + col];
        float mm = slot.x, ll = slot.y;
        merge_ml(mm, ll, m, l);
        slot = make_float2(mm, ll);
      }
    }
  };
  // One staged tile against one head's window rows.
  auto tile = [&](int start, int t, const bf16x8 (&q)[RT][NU], float (&m_)[RT], float (&l_)[RT]) {
    const int key0 = start + t * 16;
    if (key0 >= L) return;
    bf16x8 kf[NU];
    tile_frag<D>(kst, t, col, grp, kf);
    // Keys below the prefix are visible to every window row.
    const bool full = key0 + 15 < prefix;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < NU; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[u], q[rt][u], acc, 0, 0, 0);
      float s[4];
      if (full) {
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = acc[i] * p.c2;
      } else {
        const int row = rt * 16 + col;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = key0 + grp * 4 + i;
          s[i] = (j < L && j <= prefix + row) ? acc[i] * p.c2 : kNegInf;
        }
      }
      const float smax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      if (smax > m_[rt] + kRescale) {   // rare: move the reference up
        l_[rt] *= exp2_hw(m_[rt] - smax);
        m_[rt] = smax;
      }
      if (full || smax != kNegInf) {    // all masked: nothing to add (and -inf - -inf is NaN)
        float add = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) add += exp2_hw(s[i] - m_[rt]);
        l_[rt] += add;
      }
    }
  };

  // TN fully visible tiles at once: independent MFMA and exp chains
  // interleave within the wave (the compute is latency-bound otherwise).
  auto tile_multi = [&](auto tn, int start, int t, const bf16x8 (&q)[RT][NU], float (&m_)[RT], float (&l_)[RT]) {
    constexpr int TN = decltype(tn)::value;
    bf16x8 kf[TN][NU];
#pragma unroll
    for (int k = 0; k < TN; ++k) tile_frag<D>(kst, t + k, col, grp, kf[k]);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4 a[TN];
#pragma unroll
      for (int k = 0; k < TN; ++k) a[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int k = 0; k < TN; ++k) a[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[k][u], q[rt][u], a[k], 0, 0, 0);
      // exp2 against the current reference (one FMA and one exp per
      // logit); a logit far enough above it to push the tile's sum past
      // 2^64 (or the first tile, reference -inf) redoes the tile against
      // the tile's max (rare)
      auto tile_sum = [&](float m) {
        float e[TN];
#pragma unroll
        for (int k = 0; k < TN; ++k) {
          e[k] = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) e[k] += exp2_hw(fmaf(a[k][i], p.c2, -m));
        }
        float tot = 0.f;
#pragma unroll
        for (int k = 0; k < TN; ++k) tot += e[k];
        return tot;
      };
      float tot = tile_sum(m_[rt]);
      if (!(tot <= 0x1p64f)) {
        float smax = kNegInf;
#pragma unroll
        for (int k = 0; k < TN; ++k)
#pragma unroll
          for (int i = 0; i < 4; ++i) smax = fmaxf(smax, a[k][i]);
        const float mn = fmaxf(m_[rt], smax * p.c2);
        l_[rt] = m_[rt] == kNegInf ? 0.f : l_[rt] * exp2_hw(m_[rt] - mn);
        m_[rt] = mn;
        tot = tile_sum(mn);
      }
      l_[rt] += tot;
    }
  };
  auto tiles = [&](int start, int t_lo, int t_hi, const bf16x8 (&q)[RT][NU], float (&m_)[RT], float (&l_)[RT]) {
    int t = t_lo;
    constexpr int TN = KVSEL_VOTE_TN1;
    for (; t + TN - 1 < t_hi && start + t * 16 + 16 * TN - 1 < prefix; t += TN)
      tile_multi(std::integral_constant<int, TN>{}, start, t, q, m_, l_);
    for (; t < t_hi; ++t) tile(start, t, q, m_, l_);
  };

  const int pg0 = load_pages(p, b, L, c_first * kStage, c_end * kStage - 1, page_lds);
  __syncthreads();
  for (int c = c_first; c < c_end; ++c) {
    {
      uint4 buf[Stage<D>::kPer];
      stage_load<D>(p, page_lds, pg0, kvh, L, c * kStage, buf);
      __syncthreads();                       // previous chunk's readers are done
      stage_store<D>(buf, kst);
    }
    __syncthreads();
    const int start = c * kStage;
    if constexpr (PRE) {
#pragma unroll
      for (int hs = 0; hs < NS; ++hs) {
        const int g = g_lo + hs;
        if (g > g_hi) break;
        tiles(start, max(i0 - g * kTiles, 0), min(i1 - g * kTiles, kTiles), qf[hs], m_ref[hs], l_sum[hs]);
      }
    } else {
      for (int g = g_lo; g <= g_hi; ++g) {
        load_q<D, RT>(p, b, kvh * G + g, col, grp, qf[0]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) { m_ref[0][rt] = kNegInf; l_sum[0][rt] = 0.f; }
        tiles(start, max(i0 - g * kTiles, 0), min(i1 - g * kTiles, kTiles), qf[0], m_ref[0], l_sum[0]);
        flush(g, m_ref[0], l_sum[0]);
      }
    }
  }
  if constexpr (PRE) {
#pragma unroll
    for (int hs = 0; hs < NS; ++hs)
      if (g_lo + hs <= g_hi) flush(g_lo + hs, m_ref[hs], l_sum[hs]);
  }
  __syncthreads();
  // merge the waves of each (head, row) in wave order; [run][row] writes
  for (int i = tid; i < G * p.window; i += kThreads) {
    const int g = i / p.window, row = i % p.window;
    float m = kNegInf, l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float2 v = wml[(g * kWaves + w) * RT * 16 + row];
      merge_ml(m, l, v.x, v.y);
    }
    const int h = kvh * G + g;
    p.part_ml[(((size_t)b * p.num_q_heads + h) * p.n_run1 + run) * p.window + row] = make_float2(m, l);
  }
}

// Row lse (base 2) of every window row: one workgroup per (sequence, query
// head); 8 threads per row merge interleaved runs, then each other.
__global__ __launch_bounds__(256) void snapkv_lse(const float2* part_ml, const int32_t* seq_lens,
                                                  int num_q_heads, int window, int n_run, int cpw,
                                                  float* lse2) {
  const int bh = blockIdx.x;
  const int b = bh / num_q_heads;
  const int n_chunks = (seq_lens[b] + kStage - 1) / kStage;
  const int nr = (n_chunks + cpw - 1) / cpw;
  const int row = threadIdx.x / 8, part = threadIdx.x % 8;
  for (int r0 = 0; r0 < window; r0 += 32) {
    const int r = r0 + row;
    float m = kNegInf, l = 0.f;
    if (r < window) {
      const float2* ml = part_ml + (size_t)bh * n_run * window + r;
      for (int c = part; c < nr; c += 8) merge_ml(m, l, ml[(size_t)c * window].x, ml[(size_t)c * window].y);
    }
    for (int off = 1; off < 8; off *= 2) merge_ml(m, l, __shfl_xor(m, off, 8), __shfl_xor(l, off, 8));
    if (r < window && part == 0) lse2[(size_t)bh * window + r] = m + log2_hw(l);
  }
}

// Pass 2: per (run of chunks, sequence, KV head).  For each chunk: the
// staged keys are the chunk's voted keys plus the pool radius on each side;
// p = exp2(s - lse2) for every window row, column sums per head, the group
// sum in head order (or per head), the max-pool over the prefix, and the
// chunk's votes.  MFMA with the window rows as A: lane (key = key0 +
// lane%16) holds rows rt*16 + (lane/16)*4 + i, i < 4.  NHW as in pass 1
// (the rows' lse are held in registers with them).
template <int D, int RT, int NHW>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(KVSEL_VOTE_WPE2 > 0 ? KVSEL_VOTE_WPE2 : 1)))
void snapkv_pass2(VoteParams p) {
  constexpr int NU = D / 32;
  constexpr bool PRE = NHW > 0;
  constexpr int NS = PRE ? NHW : 1;
  extern __shared__ __align__(16) uint8_t sm2[];
  uint8_t* kst = sm2;                                                     // [kStage][row bytes]
  float* hv = reinterpret_cast<float*>(sm2 + kStage * Stage<D>::kRowBytes);  // [G][kStage]
  int* page_lds = reinterpret_cast<int*>(hv + (p.num_q_heads / p.num_kv_heads) * kStage);
  const int G = p.num_q_heads / p.num_kv_heads;
  const int run = blockIdx.x;
  const int b = blockIdx.y / p.num_kv_heads, kvh = blockIdx.y % p.num_kv_heads;
  const int L = p.seq_lens[b];
  const int prefix = L - p.window;
  const int c_first = run * p.cpw2;
  const int kOut = p.outc, kHalo = p.halo;
  const int c_end = min(c_first + p.cpw2, (prefix + kOut - 1) / kOut);
  if (c_first >= c_end) return;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int col = lane & 15, grp = lane >> 4;
  int i0, i1;
  wave_items(G, wave, i0, i1);
  const int g_lo = i0 / kTiles;
  const int g_hi = i0 < i1 ? (i1 - 1) / kTiles : g_lo - 1;

  bf16x8 qf[NS][RT][NU];
  float lrow[NS][RT][4];
  auto load_rows = [&](int g, bf16x8 (&q)[RT][NU], float (&lr)[RT][4]) {
    const int h = kvh * G + g;
    load_q<D, RT>(p, b, h, col, grp, q);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rt * 16 + grp * 4 + i;
        // rows past the window get +inf: exp2(s - inf) = 0
        lr[rt][i] = row < p.window ? p.lse2[((size_t)b * p.num_q_heads + h) * p.window + row] : INFINITY;
      }
  };
  if constexpr (PRE) {
#pragma unroll
    for (int hs = 0; hs < NS; ++hs)
      if (g_lo + hs <= g_hi) load_rows(g_lo + hs, qf[hs], lrow[hs]);
  }
  // Column sums of one staged tile for one head, into hv.
  auto tile = [&](int kbase, int g, int t, const bf16x8 (&q)[RT][NU], const float (&lr)[RT][4]) {
    const int key0 = kbase + t * 16;
    bf16x8 kf[NU];
    tile_frag<D>(kst, t, col, grp, kf);
    const bool full = key0 >= 0 && key0 + 15 < prefix;
    const int j = key0 + col;
    float cs = 0.f;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < NU; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q[rt][u], kf[u], acc, 0, 0, 0);
      if (full) {
#pragma unroll
        for (int i = 0; i < 4; ++i) cs += exp2_hw(fmaf(acc[i], p.c2, -lr[rt][i]));
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = rt * 16 + grp * 4 + i;
          const bool vis = j >= 0 && j < L && j <= prefix + row;
          cs += vis ? exp2_hw(fmaf(acc[i], p.c2, -lr[rt][i])) : 0.f;
        }
      }
    }
    cs = quad_rows_sum(cs);
    if (grp == 0) hv[g * kStage + t * 16 + col] = cs;
  };

  // TN fully visible tiles at once (see pass 1).
  auto tile_multi = [&](auto tn, int g, int t, const bf16x8 (&q)[RT][NU], const float (&lr)[RT][4]) {
    constexpr int TN = decltype(tn)::value;
    bf16x8 kf[TN][NU];
#pragma unroll
    for (int k = 0; k < TN; ++k) tile_frag<D>(kst, t + k, col, grp, kf[k]);
    float cs[TN];
#pragma unroll
    for (int k = 0; k < TN; ++k) cs[k] = 0.f;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4 a[TN];
#pragma unroll
      for (int k = 0; k < TN; ++k) a[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int k = 0; k < TN; ++k) a[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q[rt][u], kf[k][u], a[k], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < TN; ++k) cs[k] += exp2_hw(fmaf(a[k][i], p.c2, -lr[rt][i]));
    }
#pragma unroll
    for (int k = 0; k < TN; ++k) cs[k] = quad_rows_sum(cs[k]);
    if (grp == 0) {
#pragma unroll
      for (int k = 0; k < TN; ++k) hv[g * kStage + (t + k) * 16 + col] = cs[k];
    }
  };
  // Fully visible tiles per step: two, or four (KVSEL_VOTE_TN2) when the
  // window rows of one head are held; four measured ~1.5% faster at two
  // waves per SIMD, but need more registers than four waves per SIMD allow.
  auto tiles = [&](int kbase, int g, int t_lo, int t_hi, const bf16x8 (&q)[RT][NU], const float (&lr)[RT][4]) {
    int t = t_lo;
    if constexpr (NS == 1 && RT <= 2 && KVSEL_VOTE_TN2 == 4) {
      for (; t + 3 < t_hi; t += 4) {
        const int key0 = kbase + t * 16;
        if (key0 >= 0 && key0 + 63 < prefix) {
          tile_multi(std::integral_constant<int, 4>{}, g, t, q, lr);
        } else {
          tile(kbase, g, t, q, lr);
          tile(kbase, g, t + 1, q, lr);
          tile(kbase, g, t + 2, q, lr);
          tile(kbase, g, t + 3, q, lr);
        }
      }
    } else {
      for (; t + 1 < t_hi; t += 2) {
        const int key0 = kbase + t * 16;
        if (key0 >= 0 && key0 + 31 < prefix) {
          tile_multi(std::integral_constant<int, 2>{}, g, t, q, lr);
        } else {
          tile(kbase, g, t, q, lr);
          tile(kbase, g, t + 1, q, lr);
        }
      }
    }
    for (; t < t_hi; ++t) tile(kbase, g, t, q, lr);
  };

  const int pg0 = load_pages(p, b, L, c_first * kOut - kHalo, (c_end - 1) * kOut - kHalo + kStage - 1, page_lds);
  __syncthreads();
  for (int c = c_first; c < c_end; ++c) {
    {
      uint4 buf[Stage<D>::kPer];
      stage_load<D>(p, page_lds, pg0, kvh, L, c * kOut - kHalo, buf);
      __syncthreads();                       // previous chunk's readers are done
      stage_store<D>(buf, kst);
    }
    __syncthreads();
    const int kbase = c * kOut - kHalo;    // key of staged row 0
    if constexpr (PRE) {
#pragma unroll
      for (int hs = 0; hs < NS; ++hs) {
        const int g = g_lo + hs;
        if (g > g_hi) break;
        tiles(kbase, g, max(i0 - g * kTiles, 0), min(i1 - g * kTiles, kTiles), qf[hs], lrow[hs]);
      }
    } else {
      for (int g = g_lo; g <= g_hi; ++g) {
        load_rows(g, qf[0], lrow[0]);
        tiles(kbase, g, max(i0 - g * kTiles, 0), min(i1 - g * kTiles, kTiles), qf[0], lrow[0]);
      }
    }
    __syncthreads();
    // the group sum in head order, then the max-pool over [0, prefix)
    if (p.group_sum) {
      for (int x = tid; x < kStage; x += kThreads) {
        float v = 0.f;
        for (int g = 0; g < G; ++g) v += hv[g * kStage + x];
        hv[x] = v;
      }
      __syncthreads();
    }
    const int n_out = p.group_sum ? 1 : G;
    const int start = c * kOut;
    for (int i = tid; i < n_out * kOut; i += kThreads) {
      const int og = i / kOut, jl = i % kOut;
      const int jj = start + jl;
      if (jj >= prefix) continue;
      float best = kNegInf;
      for (int tt = max(0, jj - p.radius); tt <= min(prefix - 1, jj + p.radius); ++tt)
        best = fmaxf(best, hv[og * kStage + tt - kbase]);
      const int out_h = p.group_sum ? kvh : kvh * G + og;
      const int out_heads = p.group_sum ? p.num_kv_heads : p.num_q_heads;
      p.votes[((size_t)b * out_heads + out_h) * p.votes_stride + jj] = best;
    }
  }
}

template <int D, int RT, int NHW>
hipError_t launch_rt(const VoteParams& vp, dim3 grid1, dim3 grid2, float* lse2, float2* part_ml,
                     const int32_t* seq_lens, int B, hipStream_t s) {
  const int G = vp.num_q_heads / vp.num_kv_heads;
  const int P = 1 << vp.page_log2;
  const size_t pages1 = (size_t)vp.cpw1 * kStage / P + 2;
  const size_t pages2 = ((size_t)vp.cpw2 * vp.outc + 2 * vp.halo) / P + 2;
  const size_t lds1 = (size_t)kStage * Stage<D>::kRowBytes + (size_t)G * kWaves * RT * 16 * sizeof(float2) +
                      pages1 * sizeof(int);
  const size_t lds2 = (size_t)kStage * Stage<D>::kRowBytes + (size_t)G * kStage * sizeof(float) +
                      pages2 * sizeof(int);
  hipFuncSetAttribute(reinterpret_cast<const void*>(&snapkv_pass1<D, RT, NHW>),
                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds1);
  hipLaunchKernelGGL((snapkv_pass1<D, RT, NHW>), grid1, dim3(kThreads), lds1, s, vp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(snapkv_lse, dim3(B * vp.num_q_heads), dim3(256), 0, s, part_ml, seq_lens,
                     vp.num_q_heads, vp.window, vp.n_run1, vp.cpw1, lse2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipFuncSetAttribute(reinterpret_cast<const void*>(&snapkv_pass2<D, RT, NHW>),
                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds2);
  hipLaunchKernelGGL((snapkv_pass2<D, RT, NHW>), grid2, dim3(kThreads), lds2, s, vp);
  return hipGetLastError();
}

// Window rows held in registers for groups of <= 4 heads (one head per
// wave) and for 8 heads at windows <= 32 (two heads per wave); otherwise
// reloaded per chunk.
template <int D>
hipError_t launch_passes(const VoteParams& vp, int rt, dim3 grid1, dim3 grid2, float* lse2, float2* part_ml,
                         const int32_t* seq_lens, int B, hipStream_t s) {
  const int G = vp.num_q_heads / vp.num_kv_heads;
  const int nhw = G <= 4 ? 1 : (G == 8 && rt <= 2) ? 2 : 0;
#define KVSEL_VOTE(R, N) return launch_rt<D, R, N>(vp, grid1, grid2, lse2, part_ml, seq_lens, B, s)
  switch (rt * 4 + nhw) {
    case 4 + 1: KVSEL_VOTE(1, 1);
    case 4 + 2: KVSEL_VOTE(1, 2);
    case 4 + 0: KVSEL_VOTE(1, 0);
    case 8 + 1: KVSEL_VOTE(2, 1);
    case 8 + 2: KVSEL_VOTE(2, 2);
    case 8 + 0: KVSEL_VOTE(2, 0);
    case 12 + 1: KVSEL_VOTE(3, 1);
    case 12 + 0: KVSEL_VOTE(3, 0);
    case 16 + 1: KVSEL_VOTE(4, 1);
    case 16 + 0: KVSEL_VOTE(4, 0);
    default: return hipErrorInvalidValue;
  }
#undef KVSEL_VOTE
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Chunks per workgroup so that the grid stays near kMaxWgs workgroups.
inline int chunks_per_wg(long long rows, int n_chunks) {
  const long long total = rows * n_chunks;
  return (int)std::max<long long>(1, (total + kMaxWgs - 1) / kMaxWgs);
}

struct VotePlan {
  int cpw1, n_run1, cpw2, n_run2;
};

inline VotePlan plan_vote(int num_seqs, int num_kv_heads, int max_seq_len, int radius) {
  VotePlan v{};
  const int n1 = (max_seq_len + kStage - 1) / kStage;
  const int out2 = kStage - 2 * radius;
  const int n2 = (max_seq_len + out2 - 1) / out2;
  const long long rows = (long long)num_seqs * num_kv_heads;
  v.cpw1 = chunks_per_wg(rows, n1);
  v.n_run1 = (n1 + v.cpw1 - 1) / v.cpw1;
  v.cpw2 = chunks_per_wg(rows, n2);
  v.n_run2 = (n2 + v.cpw2 - 1) / v.cpw2;
  return v;
}

}  // namespace

size_t snapkv_workspace_bytes(int num_seqs, int num_kv_heads, int num_q_heads, int window, int max_seq_len) {
  const VotePlan v = plan_vote(num_seqs, num_kv_heads, max_seq_len, kMaxHalo);   // pass 1's layout only
  const size_t rows = (size_t)num_seqs * num_q_heads * window;
  return align256(rows * v.n_run1 * sizeof(float2)) + align256(rows * sizeof(float));
}

hipError_t launch_snapkv(const SnapkvArgs& a, hipStream_t stream) {
  const VotePlan v = plan_vote(a.num_seqs, a.num_kv_heads, a.max_seq_len, a.pool_kernel / 2);
  const size_t rows = (size_t)a.num_seqs * a.num_q_heads * a.window;
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  float2* part_ml = reinterpret_cast<float2*>(ws);
  float* lse2 = reinterpret_cast<float*>(ws + align256(rows * v.n_run1 * sizeof(float2)));
  VoteParams vp{};
  vp.k_pages = static_cast<const uint8_t*>(a.k_pages);
  vp.block_table = a.block_table;
  vp.seq_lens = a.seq_lens;
  vp.q_win = static_cast<const uint8_t*>(a.q_win);
  vp.num_kv_heads = a.num_kv_heads;
  vp.num_q_heads = a.num_q_heads;
  vp.window = a.window;
  vp.page_log2 = __builtin_ctz((unsigned)a.page_size);
  vp.max_pages = a.max_pages;
  vp.radius = a.pool_kernel / 2;
  vp.cpw1 = v.cpw1;
  vp.n_run1 = v.n_run1;
  vp.cpw2 = v.cpw2;
  vp.halo = a.pool_kernel / 2;
  vp.outc = kStage - 2 * vp.halo;
  vp.group_sum = a.group_sum;
  vp.c2 = a.scale * kLog2e;
  vp.part_ml = part_ml;
  vp.lse2 = lse2;
  vp.votes = a.votes;
  vp.votes_stride = a.votes_stride;
  const int rt = (a.window + 15) / 16;
  const dim3 grid1(v.n_run1, a.num_seqs * a.num_kv_heads);
  const dim3 grid2(v.n_run2, a.num_seqs * a.num_kv_heads);
  return a.head_dim == 128
             ? launch_passes<128>(vp, rt, grid1, grid2, lse2, part_ml, a.seq_lens, a.num_seqs, stream)
             : launch_passes<64>(vp, rt, grid1, grid2, lse2, part_ml, a.seq_lens, a.num_seqs, stream);
}

}  // namespace kvsel
