// SnapKV observation-window vote ([EVICT] "KV-cache eviction strategies",
// §4.3): the last W prompt queries (the observation window) take a causal
// softmax over the prompt's keys; each prefix key's vote is the sum of the
// probabilities it receives from the window queries of a head, optionally
// summed over the query heads of a KV group; the vote is then max-pooled
// (stride 1, same length) so the neighbours of a heavy position survive.
//
// The window logits are a real dense contraction: for one query head, the
// W x d window queries against every key.  Each 16-key x 16-row tile is one
// chain of v_mfma_f32_16x16x32_bf16 (keys as A rows, window rows as B
// columns).  One workgroup serves all G query heads of a KV head for a chunk
// of 256 keys, so the chunk is fetched from HBM once per pass and reused by
// the waves through the caches.  Two passes over K:
//   pass 1  online (max, sum of exp) of every window row over the chunk's
//           visible keys -> chunk partials, laid out [chunk][row];
//   combine per window row: lse over the chunks;
//   pass 2  recompute the tiles of the chunk plus an 8-key halo on each side,
//           p = exp(s - lse), column sums over each head's rows (16-lane DPP
//           reductions) into LDS, the group sum in head order, the max-pool,
//           and the final votes of the chunk's prefix keys.
// Every output element has one writer; there are no atomics.
#include "device_common.hpp"
#include "kvsel_internal.hpp"

namespace kvsel {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kChunk = 256;             // keys per workgroup
constexpr int kTiles = kChunk / 16;     // 16-key tiles per chunk
constexpr int kHalo = 8;                // extra keys on each side for pooling (radius <= 8)

struct VoteParams {
  const uint8_t* k_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint8_t* q_win;   // [B][Hq][W][D] bf16
  int num_kv_heads, num_q_heads, window, page_log2, max_pages, n_chunks, radius;
  bool group_sum;
  float scale;
  float2* part_ml;        // [B][Hq][n_chunks][W]
  const float* lse;       // [B][Hq][W]
  float* votes;           // [B][H_out][votes_stride]
  int64_t votes_stride;
};

__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2) {
  const float mn = fmaxf(m, m2);
  if (mn == kNegInf) return;  // both empty
  l = l * exp2_hw((m - mn) * kLog2e) + l2 * exp2_hw((m2 - mn) * kLog2e);
  m = mn;
}

// Work split inside a workgroup: the G x T (head, tile) items of the chunk
// are cut into 4 contiguous runs, one per wave, so a wave changes head (and
// reloads its window queries) at most ceil(G / 4) times.
template <int D, int RT>
__device__ __forceinline__ void load_q(const VoteParams& p, int b, int h, int col, int grp,
                                       bf16x8 (&qb)[RT][D / 32]) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rt * 16 + col;
#pragma unroll
    for (int u = 0; u < D / 32; ++u) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (row < p.window)
        w = ld16(p.q_win + ((((size_t)b * p.num_q_heads + h) * p.window + row) * D + u * 32 + grp * 8) * 2);
      qb[rt][u] = __builtin_bit_cast(bf16x8, w);
    }
  }
}

// The K rows of a workgroup's keys are staged in LDS once (all loads in
// flight together) and read back as MFMA fragments by every wave.  Rows are
// padded by 16 bytes so the 16 rows a fragment read touches fall in distinct
// banks.
template <int D>
struct Stage {
  static constexpr int kRowBytes = D * 2 + 16;
  static constexpr int kPieces = D / 8;      // 16-byte pieces per key row
};

// Stage keys kbase .. kbase + nk - 1 (clamped into [0, L)) into `kst`.
template <int D>
__device__ __forceinline__ void stage_keys(const VoteParams& p, const int* page_lds, int first_page,
                                           int b, int kvh, int L, int kbase, int nk, uint8_t* kst) {
  constexpr int PC = Stage<D>::kPieces;
  const int P = 1 << p.page_log2;
  const size_t head_stride = (size_t)P * D * 2;
  const size_t page_stride = head_stride * p.num_kv_heads;
  constexpr int kMaxPer = ((kChunk + 2 * kHalo) * PC + kThreads - 1) / kThreads;
  uint4 buf[kMaxPer];
#pragma unroll
  for (int r = 0; r < kMaxPer; ++r) {
    const int pi = threadIdx.x + r * kThreads;
    const int kl = pi / PC, seg = pi % PC;
    buf[r] = make_uint4(0, 0, 0, 0);
    if (kl < nk) {
      const int key = min(max(kbase + kl, 0), L - 1);
      const int pg = page_lds[(key >> p.page_log2) - first_page];
      buf[r] = ld16_stream(p.k_pages + (size_t)pg * page_stride + kvh * head_stride +
                           (size_t)(key & (P - 1)) * D * 2 + seg * 16);
    }
  }
#pragma unroll
  for (int r = 0; r < kMaxPer; ++r) {
    const int pi = threadIdx.x + r * kThreads;
    const int kl = pi / PC, seg = pi % PC;
    if (kl < nk) *reinterpret_cast<uint4*>(kst + kl * Stage<D>::kRowBytes + seg * 16) = buf[r];
  }
}

// MFMA A fragments of staged tile t (keys t*16 .. t*16+15 of the stage).
template <int D>
__device__ __forceinline__ void tile_frag(const uint8_t* kst, int t, int col, int grp, bf16x8 (&ka)[D / 32]) {
  const uint8_t* rp = kst + (t * 16 + col) * Stage<D>::kRowBytes + grp * 16;
#pragma unroll
  for (int u = 0; u < D / 32; ++u) ka[u] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(rp + u * 64));
}

// Logits of a loaded tile against the head's window rows: s[rt][i] for key
// key0 + grp*4 + i and row rt*16 + col, -inf where not visible.
template <int D, int RT>
__device__ __forceinline__ void tile_logits(const VoteParams& p, int L, int key0, int col, int grp,
                                            const bf16x8 (&ka)[D / 32], const bf16x8 (&qb)[RT][D / 32],
                                            float (&s)[RT][4]) {
  constexpr int NU = D / 32;
  const int prefix = L - p.window;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < NU; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[u], qb[rt][u], acc, 0, 0, 0);
    const int row = rt * 16 + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = key0 + grp * 4 + i;
      const bool vis = j >= 0 && j < L && row < p.window && j <= prefix + row;
      s[rt][i] = vis ? acc[i] * p.scale : kNegInf;
    }
  }
}

// Pass 1: per (chunk, sequence, KV head), the online (max, sum of exp) of
// every window row of every head of the group over the chunk's keys.
template <int D, int RT>
__global__ __launch_bounds__(kThreads) void snapkv_pass1(VoteParams p) {
  constexpr int NU = D / 32;
  __shared__ int page_lds[kChunk / 16 + 2];
  extern __shared__ __align__(16) uint8_t sm1[];
  uint8_t* kst = sm1;                                                    // [kChunk][row bytes]
  float2* wml = reinterpret_cast<float2*>(sm1 + kChunk * Stage<D>::kRowBytes);  // [G][kWaves][RT*16]
  const int G = p.num_q_heads / p.num_kv_heads;
  const int chunk = blockIdx.x;
  const int b = blockIdx.y / p.num_kv_heads, kvh = blockIdx.y % p.num_kv_heads;
  const int L = p.seq_lens[b];
  const int start = chunk * kChunk;
  if (start >= L) return;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int col = lane & 15, grp = lane >> 4;
  const int nk = min(kChunk, L - start);
  const int first_page = start >> p.page_log2;
  const int n_pages = ((start + nk - 1) >> p.page_log2) - first_page + 1;
  for (int i = tid; i < n_pages; i += kThreads)
    page_lds[i] = p.block_table[(size_t)b * p.max_pages + first_page + i];
  for (int i = tid; i < G * kWaves * RT * 16; i += kThreads) wml[i] = make_float2(kNegInf, 0.f);
  __syncthreads();
  stage_keys<D>(p, page_lds, first_page, b, kvh, L, start, kChunk, kst);
  __syncthreads();

  const int items = G * kTiles;
  const int per = (items + kWaves - 1) / kWaves;
  const int i0 = wave * per, i1 = min(items, i0 + per);
  int cur_h = -1;
  bf16x8 qb[RT][NU];
  float m_run[RT], l_run[RT];
  for (int it = i0; it < i1; ++it) {
    const int g = it / kTiles, t = it % kTiles;
    if (g != cur_h) {
      if (cur_h >= 0) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          for (int off = 16; off < kWave; off *= 2)
            merge_ml(m_run[rt], l_run[rt], __shfl_xor(m_run[rt], off, kWave), __shfl_xor(l_run[rt], off, kWave));
          if (grp == 0) wml[(cur_h * kWaves + wave) * RT * 16 + rt * 16 + col] = make_float2(m_run[rt], l_run[rt]);
        }
      }
      cur_h = g;
      load_q<D, RT>(p, b, kvh * G + g, col, grp, qb);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) { m_run[rt] = kNegInf; l_run[rt] = 0.f; }
    }
    bf16x8 ka[NU];
    tile_frag<D>(kst, t, col, grp, ka);
    float s[RT][4];
    tile_logits<D, RT>(p, L, start + t * 16, col, grp, ka, qb, s);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float tmax = fmaxf(fmaxf(s[rt][0], s[rt][1]), fmaxf(s[rt][2], s[rt][3]));
      const float mn = fmaxf(m_run[rt], tmax);
      if (mn != kNegInf) {
        const float ms = mn * kLog2e;
        float add = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) add += exp2_hw(fmaf(s[rt][i], kLog2e, -ms));
        l_run[rt] = l_run[rt] * exp2_hw(fmaf(m_run[rt], kLog2e, -ms)) + add;
        m_run[rt] = mn;
      }
    }
  }
  if (cur_h >= 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      for (int off = 16; off < kWave; off *= 2)
        merge_ml(m_run[rt], l_run[rt], __shfl_xor(m_run[rt], off, kWave), __shfl_xor(l_run[rt], off, kWave));
      if (grp == 0) wml[(cur_h * kWaves + wave) * RT * 16 + rt * 16 + col] = make_float2(m_run[rt], l_run[rt]);
    }
  }
  __syncthreads();
  // merge the waves of each (head, row) in wave order; coalesced [chunk][row] writes
  for (int i = tid; i < G * p.window; i += kThreads) {
    const int g = i / p.window, row = i % p.window;
    float m = kNegInf, l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float2 v = wml[(g * kWaves + w) * RT * 16 + row];
      merge_ml(m, l, v.x, v.y);
    }
    const int h = kvh * G + g;
    p.part_ml[(((size_t)b * p.num_q_heads + h) * p.n_chunks + chunk) * p.window + row] = make_float2(m, l);
  }
}

// lse of every window row: one workgroup per (sequence, query head); 8
// threads per row merge interleaved chunks, then each other.
__global__ __launch_bounds__(256) void snapkv_lse(const float2* part_ml, const int32_t* seq_lens,
                                                  int num_q_heads, int window, int n_chunks, float* lse) {
  const int bh = blockIdx.x;
  const int b = bh / num_q_heads;
  const int nc = (seq_lens[b] + kChunk - 1) / kChunk;
  const int row = threadIdx.x / 8, part = threadIdx.x % 8;
  for (int r0 = 0; r0 < window; r0 += 32) {
    const int r = r0 + row;
    float m = kNegInf, l = 0.f;
    if (r < window) {
      const float2* ml = part_ml + (size_t)bh * n_chunks * window + r;
      for (int c = part; c < nc; c += 8) merge_ml(m, l, ml[(size_t)c * window].x, ml[(size_t)c * window].y);
    }
    for (int off = 1; off < 8; off *= 2) merge_ml(m, l, __shfl_xor(m, off, 8), __shfl_xor(l, off, 8));
    if (r < window && part == 0) lse[(size_t)bh * window + r] = m + log2_hw(l) * kLn2;
  }
}

// Pass 2: per (chunk, sequence, KV head): p = exp(s - lse) for every window
// row, column sums per head over the chunk's keys plus a halo on each side,
// the group sum in head order, then the max-pool; writes the final votes of
// the chunk's prefix keys.
template <int D, int RT>
__global__ __launch_bounds__(kThreads) void snapkv_pass2(VoteParams p) {
  constexpr int NU = D / 32;
  constexpr int NK = kChunk + 2 * kHalo;               // keys with votes computed
  constexpr int NT = NK / 16;                          // tiles incl. the two halo tiles
  __shared__ int page_lds[NK / 16 + 2];
  extern __shared__ __align__(16) uint8_t sm2[];
  uint8_t* kst = sm2;                                                    // [NK][row bytes]
  float* hv = reinterpret_cast<float*>(sm2 + NK * Stage<D>::kRowBytes);  // [G][NK] per-head votes
  const int G = p.num_q_heads / p.num_kv_heads;
  const int chunk = blockIdx.x;
  const int b = blockIdx.y / p.num_kv_heads, kvh = blockIdx.y % p.num_kv_heads;
  const int L = p.seq_lens[b];
  const int prefix = L - p.window;
  const int start = chunk * kChunk;
  if (start >= prefix) return;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int col = lane & 15, grp = lane >> 4;
  const int kbase = start - kHalo;                     // key of hv[.][0]
  const int lo_key = max(kbase, 0), hi_key = min(kbase + NK, L) - 1;
  const int first_page = lo_key >> p.page_log2;
  const int n_pages = (hi_key >> p.page_log2) - first_page + 1;
  for (int i = tid; i < n_pages; i += kThreads)
    page_lds[i] = p.block_table[(size_t)b * p.max_pages + first_page + i];
  __syncthreads();
  stage_keys<D>(p, page_lds, first_page, b, kvh, L, kbase, NK, kst);
  __syncthreads();

  const int items = G * NT;
  const int per = (items + kWaves - 1) / kWaves;
  const int i0 = wave * per, i1 = min(items, i0 + per);
  int cur_h = -1;
  bf16x8 qb[RT][NU];
  float lrow[RT];
  for (int it = i0; it < i1; ++it) {
    const int g = it / NT, t = it % NT;
    if (g != cur_h) {
      cur_h = g;
      const int h = kvh * G + g;
      load_q<D, RT>(p, b, h, col, grp, qb);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int row = rt * 16 + col;
        lrow[rt] = row < p.window ? p.lse[((size_t)b * p.num_q_heads + h) * p.window + row] * kLog2e : 0.f;
      }
    }
    bf16x8 ka[NU];
    tile_frag<D>(kst, t, col, grp, ka);
    float s[RT][4];
    tile_logits<D, RT>(p, L, kbase + t * 16, col, grp, ka, qb, s);
    float cs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) cs[i] += exp2_hw(fmaf(s[rt][i], kLog2e, -lrow[rt]));
#pragma unroll
    for (int i = 0; i < 4; ++i) cs[i] = group_sum<16>(cs[i]);
    if (col == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) hv[g * NK + t * 16 + grp * 4 + i] = cs[i];
    }
  }
  __syncthreads();
  // group sum (head order) or per head, then the max-pool over [0, prefix)
  const int n_out = p.group_sum ? 1 : G;
  for (int i = tid; i < n_out * kChunk; i += kThreads) {
    const int og = i / kChunk, jl = i % kChunk;
    const int j = start + jl;
    if (j >= prefix) continue;
    float best = kNegInf;
    for (int t = max(0, j - p.radius); t <= min(prefix - 1, j + p.radius); ++t) {
      const int x = t - kbase;
      float v;
      if (p.group_sum) {
        v = 0.f;
        for (int g = 0; g < G; ++g) v += hv[g * NK + x];
      } else {
        v = hv[og * NK + x];
      }
      best = fmaxf(best, v);
    }
    const int out_h = p.group_sum ? kvh : kvh * G + og;
    const int out_heads = p.group_sum ? p.num_kv_heads : p.num_q_heads;
    p.votes[((size_t)b * out_heads + out_h) * p.votes_stride + j] = best;
  }
}

template <int D>
hipError_t launch_passes(const VoteParams& vp, int rt, dim3 grid, float* lse, float2* part_ml,
                         const int32_t* seq_lens, int B, hipStream_t s) {
  const int G = vp.num_q_heads / vp.num_kv_heads;
  const size_t lds1 = (size_t)kChunk * Stage<D>::kRowBytes + (size_t)G * kWaves * rt * 16 * sizeof(float2);
  const size_t lds2 = (size_t)(kChunk + 2 * kHalo) * Stage<D>::kRowBytes +
                      (size_t)G * (kChunk + 2 * kHalo) * sizeof(float);
#define KVSEL_P1(R)                                                                              \
  hipFuncSetAttribute(reinterpret_cast<const void*>(&snapkv_pass1<D, R>),                       \
                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds1);                    \
  hipLaunchKernelGGL((snapkv_pass1<D, R>), grid, dim3(kThreads), lds1, s, vp)
#define KVSEL_P2(R)                                                                              \
  hipFuncSetAttribute(reinterpret_cast<const void*>(&snapkv_pass2<D, R>),                       \
                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds2);                    \
  hipLaunchKernelGGL((snapkv_pass2<D, R>), grid, dim3(kThreads), lds2, s, vp)
  switch (rt) {
    case 1: KVSEL_P1(1); break;
    case 2: KVSEL_P1(2); break;
    case 3: KVSEL_P1(3); break;
    case 4: KVSEL_P1(4); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(snapkv_lse, dim3(B * vp.num_q_heads), dim3(256), 0, s, part_ml, seq_lens,
                     vp.num_q_heads, vp.window, vp.n_chunks, lse);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (rt) {
    case 1: KVSEL_P2(1); break;
    case 2: KVSEL_P2(2); break;
    case 3: KVSEL_P2(3); break;
    case 4: KVSEL_P2(4); break;
    default: return hipErrorInvalidValue;
  }
#undef KVSEL_P1
#undef KVSEL_P2
  return hipGetLastError();
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

size_t snapkv_workspace_bytes(int num_seqs, int num_q_heads, int window, int max_seq_len) {
  const int n_chunks = (max_seq_len + kChunk - 1) / kChunk;
  const size_t rows = (size_t)num_seqs * num_q_heads * window;
  return align256(rows * n_chunks * sizeof(float2)) + align256(rows * sizeof(float));
}

hipError_t launch_snapkv(const SnapkvArgs& a, hipStream_t stream) {
  const int n_chunks = (a.max_seq_len + kChunk - 1) / kChunk;
  const size_t rows = (size_t)a.num_seqs * a.num_q_heads * a.window;
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  float2* part_ml = reinterpret_cast<float2*>(ws);
  float* lse = reinterpret_cast<float*>(ws + align256(rows * n_chunks * sizeof(float2)));
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
  vp.n_chunks = n_chunks;
  vp.radius = a.pool_kernel / 2;
  vp.group_sum = a.group_sum;
  vp.scale = a.scale;
  vp.part_ml = part_ml;
  vp.lse = lse;
  vp.votes = a.votes;
  vp.votes_stride = a.votes_stride;
  const int rt = (a.window + 15) / 16;
  const dim3 grid(n_chunks, a.num_seqs * a.num_kv_heads);
  return a.head_dim == 128 ? launch_passes<128>(vp, rt, grid, lse, part_ml, a.seq_lens, a.num_seqs, stream)
                           : launch_passes<64>(vp, rt, grid, lse, part_ml, a.seq_lens, a.num_seqs, stream);
}

}  // namespace kvsel
