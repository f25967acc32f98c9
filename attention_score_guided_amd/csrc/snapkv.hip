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
// columns).  Two passes over K:
//   pass 1  per (head, 256-key chunk): online (max, sum of exp) of every
//           window row over the chunk's visible keys -> chunk partials;
//   combine per window row: lse over the chunks;
//   pass 2  per (head, chunk of prefix keys): recompute the tile,
//           p = exp(s - lse), column sums over the head's rows (16-lane DPP
//           reductions) -> per-head votes;
//   pool    per output: sum the group's heads in head order, max over the
//           pooling window.
// Every output element has one writer; there are no atomics.
#include "device_common.hpp"
#include "kvsel_internal.hpp"

namespace kvsel {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kChunk = 256;             // keys per workgroup: 4 waves x 4 tiles of 16
constexpr int kTilesPerWave = kChunk / (16 * kWaves);

struct VoteParams {
  const uint8_t* k_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint8_t* q_win;   // [B][Hq][W][D] bf16
  int num_kv_heads, num_q_heads, window, page_log2, max_pages, n_chunks;
  float scale;
  float2* part_ml;        // [B][Hq][W][n_chunks]
  const float* lse;       // [B][Hq][W]
  float* head_votes;      // [B][Hq][hv_stride]
  int64_t hv_stride;
};

__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2) {
  const float mn = fmaxf(m, m2);
  if (mn == kNegInf) return;  // both empty
  l = l * exp2_hw((m - mn) * kLog2e) + l2 * exp2_hw((m2 - mn) * kLog2e);
  m = mn;
}

template <int D, int RT, int PASS>
__global__ __launch_bounds__(kThreads) void snapkv_pass(VoteParams p) {
  constexpr int NU = D / 32;
  __shared__ int page_lds[kChunk / 16 + 2];
  __shared__ float2 wml[kWaves][RT * 16];

  const int G = p.num_q_heads / p.num_kv_heads;
  const int g = blockIdx.x;
  const int chunk = blockIdx.y;
  const int b = blockIdx.z / p.num_kv_heads;
  const int kvh = blockIdx.z % p.num_kv_heads;
  const int h = kvh * G + g;
  const int L = p.seq_lens[b];
  const int W = p.window;
  const int prefix = L - W;
  const int start = chunk * kChunk;
  const int limit = PASS == 1 ? L : prefix;   // pass 2 only votes for prefix keys
  if (start >= limit) return;
  const int n_keys = min(kChunk, limit - start);
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int col = lane & 15, grp = lane >> 4;
  const int P = 1 << p.page_log2;
  const int first_page = start >> p.page_log2;
  const int n_pages = ((start + n_keys - 1) >> p.page_log2) - first_page + 1;
  for (int i = tid; i < n_pages; i += kThreads)
    page_lds[i] = p.block_table[(size_t)b * p.max_pages + first_page + i];

  // B operand: Q_win^T, column = window row rt*16 + col (zero past W).
  bf16x8 qb[RT][NU];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rt * 16 + col;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (row < W) w = ld16(p.q_win + ((((size_t)b * p.num_q_heads + h) * W + row) * D + u * 32 + grp * 8) * 2);
      qb[rt][u] = __builtin_bit_cast(bf16x8, w);
    }
  }
  float lse_row[RT];
  if constexpr (PASS == 2) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = rt * 16 + col;
      lse_row[rt] = row < W ? p.lse[((size_t)b * p.num_q_heads + h) * W + row] * kLog2e : 0.f;
    }
  }
  __syncthreads();

  const size_t head_stride = (size_t)P * D * 2;
  const size_t page_stride = head_stride * p.num_kv_heads;
  float m_run[RT], l_run[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) { m_run[rt] = kNegInf; l_run[rt] = 0.f; }

  bf16x8 ka[kTilesPerWave][NU];
#pragma unroll
  for (int t = 0; t < kTilesPerWave; ++t) {
    const int kl = min(wave * kTilesPerWave * 16 + t * 16 + col, n_keys - 1);
    const int j = start + kl;
    const int pg = page_lds[(j >> p.page_log2) - first_page];
    const uint8_t* rp = p.k_pages + (size_t)pg * page_stride + kvh * head_stride +
                        (size_t)(j & (P - 1)) * D * 2 + grp * 16;
#pragma unroll
    for (int u = 0; u < NU; ++u) ka[t][u] = __builtin_bit_cast(bf16x8, ld16_stream(rp + u * 64));
  }
#pragma unroll
  for (int t = 0; t < kTilesPerWave; ++t) {
    const int k0 = wave * kTilesPerWave * 16 + t * 16 + grp * 4;   // chunk-local key of acc[0]
    float colsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < NU; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[t][u], qb[rt][u], acc, 0, 0, 0);
      const int row = rt * 16 + col;
      float s[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = start + k0 + i;
        // visible: a real key, a real window row, causal (j <= L - W + row)
        const bool vis = (k0 + i < n_keys) && row < W && j <= prefix + row;
        s[i] = vis ? acc[i] * p.scale : kNegInf;
      }
      if constexpr (PASS == 1) {
        const float tmax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        const float mn = fmaxf(m_run[rt], tmax);
        if (mn != kNegInf) {
          const float ms = mn * kLog2e;
          float add = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) add += exp2_hw(fmaf(s[i], kLog2e, -ms));
          l_run[rt] = l_run[rt] * exp2_hw(fmaf(m_run[rt], kLog2e, -ms)) + add;
          m_run[rt] = mn;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) colsum[i] += exp2_hw(fmaf(s[i], kLog2e, -lse_row[rt]));
      }
    }
    if constexpr (PASS == 2) {
      // sum over the 16 window rows held by the lanes of this DPP row
#pragma unroll
      for (int i = 0; i < 4; ++i) colsum[i] = group_sum<16>(colsum[i]);
      if (col == 0) {
        float* hv = p.head_votes + ((size_t)b * p.num_q_heads + h) * p.hv_stride + start;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (k0 + i < n_keys) hv[k0 + i] = colsum[i];
      }
    }
  }

  if constexpr (PASS == 1) {
    // merge the key groups (lanes 16 apart hold other keys of the same rows)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      for (int off = 16; off < kWave; off *= 2) {
        const float m2 = __shfl_xor(m_run[rt], off, kWave);
        const float l2 = __shfl_xor(l_run[rt], off, kWave);
        merge_ml(m_run[rt], l_run[rt], m2, l2);
      }
      if (grp == 0) wml[wave][rt * 16 + col] = make_float2(m_run[rt], l_run[rt]);
    }
    __syncthreads();
    if (tid < W) {
      float m = kNegInf, l = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) merge_ml(m, l, wml[w][tid].x, wml[w][tid].y);
      p.part_ml[(((size_t)b * p.num_q_heads + h) * W + tid) * p.n_chunks + chunk] = make_float2(m, l);
    }
  }
}

// lse of every window row from its chunk partials (chunks past the row's
// last visible key were not launched or hold (-inf, 0)).
__global__ __launch_bounds__(256) void snapkv_lse(const float2* part_ml, const int32_t* seq_lens,
                                                  int num_q_heads, int window, int n_chunks,
                                                  int total_rows, float* lse) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= total_rows) return;
  const int b = r / (num_q_heads * window);
  const int L = seq_lens[b];
  const int nc = (L + kChunk - 1) / kChunk;
  float m = kNegInf, l = 0.f;
  const float2* ml = part_ml + (size_t)r * n_chunks;
  for (int c = 0; c < nc; ++c) merge_ml(m, l, ml[c].x, ml[c].y);
  lse[r] = m + log2_hw(l) * kLn2;
}

// votes[b][g][j] = max over |t| <= r of v(j + t), v = head vote summed over the
// group (SUM) or the head's own vote (NONE); j < L - W; padding ignored.
__global__ __launch_bounds__(256) void snapkv_pool(const float* head_votes, int64_t hv_stride,
                                                   const int32_t* seq_lens, int num_q_heads,
                                                   int num_out_heads, int group, int window,
                                                   int radius, float* votes, int64_t votes_stride) {
  const int b = blockIdx.z, og = blockIdx.y;
  const int n = seq_lens[b] - window;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= n) return;
  const int h0 = og * group;
  const float* hv = head_votes + ((size_t)b * num_q_heads + h0) * hv_stride;
  float best = kNegInf;
  for (int t = max(0, j - radius); t <= min(n - 1, j + radius); ++t) {
    float v = 0.f;
    for (int gg = 0; gg < group; ++gg) v += hv[(size_t)gg * hv_stride + t];
    best = fmaxf(best, v);
  }
  votes[((size_t)b * num_out_heads + og) * votes_stride + j] = best;
}

template <int D, int RT, int PASS>
void launch_pass(const VoteParams& vp, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((snapkv_pass<D, RT, PASS>), grid, dim3(kThreads), 0, s, vp);
}

template <int D, int PASS>
hipError_t launch_pass_rt(const VoteParams& vp, int rt, dim3 grid, hipStream_t s) {
  switch (rt) {
    case 1: launch_pass<D, 1, PASS>(vp, grid, s); break;
    case 2: launch_pass<D, 2, PASS>(vp, grid, s); break;
    case 3: launch_pass<D, 3, PASS>(vp, grid, s); break;
    case 4: launch_pass<D, 4, PASS>(vp, grid, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

size_t snapkv_workspace_bytes(int num_seqs, int num_q_heads, int window, int max_seq_len) {
  const int n_chunks = (max_seq_len + kChunk - 1) / kChunk;
  const size_t rows = (size_t)num_seqs * num_q_heads * window;
  return align256(rows * n_chunks * sizeof(float2)) + align256(rows * sizeof(float)) +
         align256((size_t)num_seqs * num_q_heads * max_seq_len * sizeof(float));
}

hipError_t launch_snapkv(const SnapkvArgs& a, hipStream_t stream) {
  const int n_chunks = (a.max_seq_len + kChunk - 1) / kChunk;
  const size_t rows = (size_t)a.num_seqs * a.num_q_heads * a.window;
  uint8_t* ws = static_cast<uint8_t*>(a.workspace);
  float2* part_ml = reinterpret_cast<float2*>(ws);
  float* lse = reinterpret_cast<float*>(ws + align256(rows * n_chunks * sizeof(float2)));
  float* head_votes = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(lse) + align256(rows * sizeof(float)));
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
  vp.scale = a.scale;
  vp.part_ml = part_ml;
  vp.lse = lse;
  vp.head_votes = head_votes;
  vp.hv_stride = a.max_seq_len;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int rt = (a.window + 15) / 16;
  const dim3 grid(G, n_chunks, a.num_seqs * a.num_kv_heads);
  hipError_t e = a.head_dim == 128 ? launch_pass_rt<128, 1>(vp, rt, grid, stream)
                                   : launch_pass_rt<64, 1>(vp, rt, grid, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(snapkv_lse, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream, part_ml,
                     a.seq_lens, a.num_q_heads, a.window, n_chunks, (int)rows, lse);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = a.head_dim == 128 ? launch_pass_rt<128, 2>(vp, rt, grid, stream)
                        : launch_pass_rt<64, 2>(vp, rt, grid, stream);
  if (e != hipSuccess) return e;
  const int out_heads = a.group_sum ? a.num_kv_heads : a.num_q_heads;
  const dim3 pgrid((a.max_seq_len + 255) / 256, out_heads, a.num_seqs);
  hipLaunchKernelGGL(snapkv_pool, pgrid, dim3(256), 0, stream, head_votes, (int64_t)a.max_seq_len,
                     a.seq_lens, a.num_q_heads, out_heads, a.group_sum ? G : 1, a.window,
                     a.pool_kernel / 2, a.votes, a.votes_stride);
  return hipGetLastError();
}

}  // namespace kvsel
