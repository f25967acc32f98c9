// FP8 indexer scores ([LONGCTX] "Long context, KV eviction and sparse
// attention", sparse-attention section: a lightweight indexer scores every
// cached token with few heads in FP8, and each query attends only to the
// top-scoring 2048 tokens).
//
// scores[b][h][j] = scale * q[b][h] . k[b][h / G][j] for j < L_b, with q and
// the indexer keys stored as FP8 E4M3 (OCP: bias 7, no infinities, max 448)
// and the products accumulated in fp32 on the matrix cores
// (v_mfma_f32_16x16x32_fp8_fp8).  Products of two E4M3 values are exact in
// fp32, so the only rounding is the fp32 accumulation.
//
// indexer_fp8_kernel: grid (chunk of keys, KV head x head group, sequence).
// A wave owns a run of 16-key tiles; a lane loads the 16-byte (d = 64) or
// 32-byte (d = 128) piece of one key row that feeds its operand slots, so a
// tile is one fully coalesced 1 KB (or 2 KB) read.  The dot product is a sum
// over the channels, so any assignment of channels to MFMA k-slots that A
// (keys) and B (queries) share gives the same products: lane group g takes
// channels [g * D/4, (g + 1) * D/4) and feeds them to the k-steps in order.
// Up to 32 query heads (two 16-column B tiles) share each K tile.
#include "device_common.hpp"
#include "kvsel_internal.hpp"

namespace kvsel {

namespace {

constexpr int kIThreads = 256;
constexpr int kIWaves = kIThreads / kWave;
constexpr int kIMaxChunk = 1024;

struct IndexerParams {
  const uint8_t* k_pages;     // [num_pages][H_kv][P][D] E4M3
  const int32_t* block_table;
  const int32_t* seq_lens;
  const uint8_t* q;           // [B][H_q][D] E4M3
  float* scores;              // [B][H_q][stride]
  int64_t stride;
  int num_kv_heads, num_q_heads, group, hgroups, page_log2, max_pages, chunk;
  float scale;
};

// ALIGNED: every score row is 16-byte aligned (checked on the host), so whole
// chunks take 16-byte stores; otherwise every tile goes through a per-wave
// LDS slice and is written as runs of 16 consecutive keys.
template <int D, int NCT, bool ALIGNED>
__global__ __launch_bounds__(kIThreads) void indexer_fp8_kernel(IndexerParams p) {
  constexpr int NU = D / 32;          // k-steps of 32 channels
  constexpr int BPL = D / 4;          // bytes of a key row per lane (16 or 32)
  constexpr int QB = 4;               // tiles whose loads are issued together
  constexpr int GTL = 16 * NCT;
  __shared__ int page_lds[kIMaxChunk / 16 + 2];
  __shared__ float sc_stage[ALIGNED ? 1 : kIWaves][16 * 16];   // per wave: one tile, [head slot][key]
  const int C = p.chunk;
  const int kvh = blockIdx.y / p.hgroups, hg = blockIdx.y % p.hgroups, b = blockIdx.z;
  const int L = p.seq_lens[b];
  const int start = blockIdx.x * C;
  if (start >= L) return;
  const int n_keys = min(C, L - start);
  const int n_heads = min(GTL, p.group - hg * GTL);
  const int h0 = kvh * p.group + hg * GTL;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int col = lane & 15, grp = lane >> 4;
  const int P = 1 << p.page_log2;
  const int first_page = start >> p.page_log2;
  const int n_pages = ((start + n_keys - 1) >> p.page_log2) - first_page + 1;
  for (int i = tid; i < n_pages; i += kIThreads) page_lds[i] = p.block_table[(size_t)b * p.max_pages + first_page + i];
  // B operand: column = head, the lane's channels [grp * BPL, (grp + 1) * BPL)
  long qb[NCT][NU];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int hh = ct * 16 + col;
    const uint8_t* qp = p.q + ((size_t)b * p.num_q_heads + h0 + hh) * D + grp * BPL;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      qb[ct][u] = 0;
      if (hh < n_heads) qb[ct][u] = *reinterpret_cast<const long*>(qp + u * 8);
    }
  }
  __syncthreads();
  const size_t head_stride = (size_t)P * D;
  const size_t page_stride = head_stride * p.num_kv_heads;
  auto krow = [&](int key) -> const uint8_t* {
    const int j = start + key;
    const int pg = page_lds[(j >> p.page_log2) - first_page];
    return p.k_pages + (size_t)pg * page_stride + kvh * head_stride + (size_t)(j & (P - 1)) * D;
  };
  const int per_wave = C / kIWaves;
  const int nt = per_wave / 16;
  const int wbase = wave * per_wave;
  const bool vec = ALIGNED && n_keys == C;
  for (int t0 = 0; t0 < nt; t0 += QB) {
    uint4 kr[QB][BPL / 16];
#pragma unroll
    for (int t = 0; t < QB; ++t) {
      const uint8_t* rp = krow(min(wbase + min(t0 + t, nt - 1) * 16 + col, n_keys - 1)) + grp * BPL;
#pragma unroll
      for (int v = 0; v < BPL / 16; ++v) kr[t][v] = ld16_stream(rp + v * 16);
    }
#pragma unroll
    for (int t = 0; t < QB; ++t) {
      if (t0 + t >= nt) continue;
      long ka[NU];
#pragma unroll
      for (int v = 0; v < BPL / 16; ++v) {
        ka[2 * v] = (long)kr[t][v].x | ((long)kr[t][v].y << 32);
        ka[2 * v + 1] = (long)kr[t][v].z | ((long)kr[t][v].w << 32);
      }
      const int k0 = wbase + (t0 + t) * 16 + grp * 4;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < NU; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(ka[u], qb[ct][u], acc, 0, 0, 0);
        const int hh = ct * 16 + col;
        if constexpr (ALIGNED) {
          if (hh < n_heads) {
            float* out = p.scores + ((size_t)b * p.num_q_heads + h0 + hh) * p.stride + start;
            if (vec) {
              *reinterpret_cast<float4*>(out + k0) =
                  make_float4(acc[0] * p.scale, acc[1] * p.scale, acc[2] * p.scale, acc[3] * p.scale);
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (k0 + i < n_keys) out[k0 + i] = acc[i] * p.scale;
            }
          }
        } else {
          // Unaligned rows: through this wave's LDS slice, so a store instruction writes runs of 16 consecutive
          // keys (4 heads x 16 keys).  One wave's LDS operations complete in
          // order; the barriers pin the compiler's ordering.
          float* sl = sc_stage[wave];
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
              p.scores[((size_t)b * p.num_q_heads + h0 + ct * 16 + hl) * p.stride + start + key] = sl[hl * 16 + col];
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
        }
      }
    }
  }
}

template <int D, int NCT>
void launch_fp8(bool aligned, dim3 grid, hipStream_t stream, const IndexerParams& ip) {
  if (aligned) hipLaunchKernelGGL((indexer_fp8_kernel<D, NCT, true>), grid, dim3(kIThreads), 0, stream, ip);
  else hipLaunchKernelGGL((indexer_fp8_kernel<D, NCT, false>), grid, dim3(kIThreads), 0, stream, ip);
}

}  // namespace

hipError_t launch_indexer_fp8(const void* k_pages, const int32_t* block_table, const int32_t* seq_lens,
                              const void* q, int num_seqs, int num_kv_heads, int num_q_heads, int head_dim,
                              int page_size, int max_pages, int max_seq_len, float scale, float* scores,
                              int64_t stride, hipStream_t stream) {
  IndexerParams ip{};
  ip.k_pages = static_cast<const uint8_t*>(k_pages);
  ip.block_table = block_table;
  ip.seq_lens = seq_lens;
  ip.q = static_cast<const uint8_t*>(q);
  ip.scores = scores;
  ip.stride = stride;
  ip.num_kv_heads = num_kv_heads;
  ip.num_q_heads = num_q_heads;
  ip.group = num_q_heads / num_kv_heads;
  const int nct = ip.group > 16 ? 2 : 1;
  ip.hgroups = (ip.group + 16 * nct - 1) / (16 * nct);
  ip.page_log2 = __builtin_ctz((unsigned)page_size);
  ip.max_pages = max_pages;
  ip.scale = scale;
  // the largest chunk (<= 1024 keys, >= 128) that still gives >= 1024 workgroups
  int chunk = kIMaxChunk;
  while (chunk > 128 && (long long)num_seqs * num_kv_heads * ip.hgroups * ((max_seq_len + chunk - 1) / chunk) < 1024)
    chunk /= 2;
  ip.chunk = chunk;
  const dim3 grid((max_seq_len + chunk - 1) / chunk, num_kv_heads * ip.hgroups, num_seqs);
  const bool al = (ip.stride & 3) == 0 && (reinterpret_cast<uintptr_t>(ip.scores) & 15) == 0;
  if (head_dim == 128) {
    if (nct == 2) launch_fp8<128, 2>(al, grid, stream, ip);
    else launch_fp8<128, 1>(al, grid, stream, ip);
  } else {
    if (nct == 2) launch_fp8<64, 2>(al, grid, stream, ip);
    else launch_fp8<64, 1>(al, grid, stream, ip);
  }
  return hipGetLastError();
}

}  // namespace kvsel
