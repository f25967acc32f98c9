// Standalone H2O accumulation and token-to-block aggregation.
//
// accumulate:      [EVICT] "KV-cache eviction strategies", §4.2 (H2O adds each
//                  step's attention weights to a per-position cumulative score);
//                  decay < 1 is the exponential decay of [OFFLOAD] §2.1.
// block_aggregate: [OFFLOAD] "Sparse attention x KV-cache offloading", §3.1
//                  (max and mean of the token scores inside a block) and §5.1
//                  (one fp32 score per block); the head sum and the
//                  accumulate-into-output mode give one score per block across
//                  KV heads and layers.
// Both are streaming, HBM-bound passes with one writer per output element.
#include "device_common.hpp"
#include "kvsel_internal.hpp"

namespace kvsel {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void accumulate_kernel(
    const float* __restrict__ probs, int64_t probs_stride, const int32_t* __restrict__ seq_lens,
    int num_q_heads, int num_kv_heads, int keys_per_block, float decay, float* __restrict__ cum,
    int64_t cum_stride) {
  const int b = blockIdx.z, c = blockIdx.y;
  const int L = seq_lens[b];
  const int start = blockIdx.x * keys_per_block;
  if (start >= L) return;
  const int end = min(L, start + keys_per_block);
  const int G = num_q_heads / num_kv_heads;
  const float* pr = probs + ((size_t)b * num_q_heads + (size_t)c * G) * probs_stride;
  float* cp = cum + ((size_t)b * num_kv_heads + c) * cum_stride;
  for (int j = start + threadIdx.x; j < end; j += kThreads) {
    float acc = 0.f;
    for (int g = 0; g < G; ++g) acc += pr[(size_t)g * probs_stride + j];
    cp[j] = fmaf(decay, cp[j], acc);
  }
}

// Vectorised block aggregation: each thread owns 4 consecutive positions of a
// row; TPB = block_size / 4 threads share one block (TPB in 1..64, a power of
// two), so a block's max and sum are reduced across an aligned lane group.
// One workgroup covers 1024 positions of one sequence and either one head
// (head_sum = false) or all heads summed in head order (head_sum = true).
template <int TPB>
__global__ __launch_bounds__(kThreads) void block_agg_vec(
    const float* __restrict__ scores, int64_t score_stride, const int32_t* __restrict__ seq_lens,
    int num_heads, int block_size, bool head_sum, bool accumulate, float* __restrict__ out_max,
    float* __restrict__ out_mean, int64_t out_stride, int64_t out_seq_stride) {
  const int b = head_sum ? blockIdx.y : blockIdx.y / num_heads;
  const int hsel = head_sum ? 0 : blockIdx.y % num_heads;
  const int L = seq_lens[b];
  const int pos = blockIdx.x * 1024 + threadIdx.x * 4;
  const int blk = pos / block_size;
  const int n_blk = (L + block_size - 1) / block_size;
  if (blockIdx.x * 1024 >= L) return;
  const int h_begin = head_sum ? 0 : hsel;
  const int h_end = head_sum ? num_heads : hsel + 1;
  float mx_tot = 0.f, mean_tot = 0.f;
  const int count = min(block_size, L - blk * block_size);
  for (int h = h_begin; h < h_end; ++h) {
    const float* row = scores + ((size_t)b * num_heads + h) * score_stride;
    float mx = kNegInf, sm = 0.f;
    if (pos < L) {
      if (pos + 3 < L) {
        const float4 v = *reinterpret_cast<const float4*>(row + pos);
        mx = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
        sm = (v.x + v.y) + (v.z + v.w);
      } else {
        for (int t = pos; t < L; ++t) {
          mx = fmaxf(mx, row[t]);
          sm += row[t];
        }
      }
    }
    mx = group_max<TPB>(mx);
    sm = group_sum<TPB>(sm);
    mx_tot += mx;
    mean_tot += sm / (float)count;
  }
  if (threadIdx.x % TPB != 0 || blk >= n_blk) return;
  const size_t o = (size_t)b * out_seq_stride + (head_sum ? 0 : (size_t)hsel * out_stride) + blk;
  if (out_max) out_max[o] = accumulate ? out_max[o] + mx_tot : mx_tot;
  if (out_mean) out_mean[o] = accumulate ? out_mean[o] + mean_tot : mean_tot;
}

// Any block size: one thread per (row, block), sequential over the block.
__global__ __launch_bounds__(kThreads) void block_agg_generic(
    const float* __restrict__ scores, int64_t score_stride, const int32_t* __restrict__ seq_lens,
    int num_seqs, int num_heads, int n_blk_max, int block_size, bool head_sum, bool accumulate,
    float* __restrict__ out_max, float* __restrict__ out_mean, int64_t out_stride, int64_t out_seq_stride) {
  const int rows = head_sum ? num_seqs : num_seqs * num_heads;
  const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= (long long)rows * n_blk_max) return;
  const int r = (int)(gid / n_blk_max);
  const int blk = (int)(gid % n_blk_max);
  const int b = head_sum ? r : r / num_heads;
  const int L = seq_lens[b];
  if (blk * block_size >= L) return;
  const int lo = blk * block_size, hi = min(L, lo + block_size);
  const int h_begin = head_sum ? 0 : r % num_heads;
  const int h_end = head_sum ? num_heads : h_begin + 1;
  float mx_tot = 0.f, mean_tot = 0.f;
  for (int h = h_begin; h < h_end; ++h) {
    const float* row = scores + ((size_t)b * num_heads + h) * score_stride;
    float mx = kNegInf, sm = 0.f;
    for (int t = lo; t < hi; ++t) {
      mx = fmaxf(mx, row[t]);
      sm += row[t];
    }
    mx_tot += mx;
    mean_tot += sm / (float)(hi - lo);
  }
  const size_t o = (size_t)b * out_seq_stride + (head_sum ? 0 : (size_t)(r % num_heads) * out_stride) + blk;
  if (out_max) out_max[o] = accumulate ? out_max[o] + mx_tot : mx_tot;
  if (out_mean) out_mean[o] = accumulate ? out_mean[o] + mean_tot : mean_tot;
}

// Block size 1 summed over heads: a column sum of [B][H][stride] rows, e.g.
// per-layer block scores stacked as extra heads.  A workgroup owns 64
// columns of one sequence; its 16 waves split the heads, then LDS adds the
// 16 partial sums in a fixed order.
constexpr int kColWaves = 16;
__global__ __launch_bounds__(64 * kColWaves) void head_sum_columns(
    const float* __restrict__ scores, int64_t score_stride, const int32_t* __restrict__ seq_lens,
    int num_heads, int max_len, bool accumulate, float* __restrict__ out_max,
    float* __restrict__ out_mean, int64_t out_seq_stride) {
  __shared__ float part[kColWaves][64];
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = blockIdx.x * 64 + lane;
  const bool live = col < min(seq_lens[b], max_len);
  float acc = 0.f;
  if (live) {
    const float* p = scores + (size_t)b * num_heads * score_stride + col;
#pragma unroll 8
    for (int h = w; h < num_heads; h += kColWaves)
      acc += __builtin_nontemporal_load(p + (size_t)h * score_stride);
  }
  part[w][lane] = acc;
  __syncthreads();
  if (w == 0 && live) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kColWaves; ++i) s += part[i][lane];
    const size_t o = (size_t)b * out_seq_stride + col;
    if (out_max) out_max[o] = accumulate ? out_max[o] + s : s;
    if (out_mean) out_mean[o] = accumulate ? out_mean[o] + s : s;
  }
}

}  // namespace

hipError_t launch_accumulate(const float* probs, int64_t probs_stride, const int32_t* seq_lens,
                             int num_seqs, int num_q_heads, int num_kv_heads, int max_seq_len,
                             float decay, float* cum, int64_t cum_stride, hipStream_t stream) {
  const int kpb = 1024;
  const dim3 grid((max_seq_len + kpb - 1) / kpb, num_kv_heads, num_seqs);
  hipLaunchKernelGGL(accumulate_kernel, grid, dim3(kThreads), 0, stream, probs, probs_stride,
                     seq_lens, num_q_heads, num_kv_heads, kpb, decay, cum, cum_stride);
  return hipGetLastError();
}

hipError_t launch_block_aggregate(const float* scores, int64_t score_stride,
                                  const int32_t* seq_lens, int num_seqs, int num_heads,
                                  int max_seq_len, int block_size, bool head_sum, bool accumulate,
                                  float* out_max, float* out_mean, int64_t out_stride,
                                  int64_t out_seq_stride, hipStream_t stream) {
  if (out_seq_stride <= 0) out_seq_stride = head_sum ? out_stride : (int64_t)num_heads * out_stride;
  const bool pow2 = (block_size & (block_size - 1)) == 0;
  const bool vec_ok = pow2 && block_size >= 4 && block_size <= 256 && score_stride % 4 == 0 &&
                      (reinterpret_cast<uintptr_t>(scores) & 15) == 0;
  if (vec_ok) {
    const dim3 grid((max_seq_len + 1023) / 1024, head_sum ? num_seqs : num_seqs * num_heads);
    const int tpb = block_size / 4;
#define KVSEL_AGG(T)                                                                       \
  case T:                                                                                  \
    hipLaunchKernelGGL(block_agg_vec<T>, grid, dim3(kThreads), 0, stream, scores,          \
                       score_stride, seq_lens, num_heads, block_size, head_sum, accumulate, \
                       out_max, out_mean, out_stride, out_seq_stride);                     \
    break;
    switch (tpb) {
      KVSEL_AGG(1)
      KVSEL_AGG(2)
      KVSEL_AGG(4)
      KVSEL_AGG(8)
      KVSEL_AGG(16)
      KVSEL_AGG(32)
      KVSEL_AGG(64)
      default: return hipErrorInvalidValue;
    }
#undef KVSEL_AGG
    return hipGetLastError();
  }
  if (block_size == 1 && head_sum) {
    const dim3 grid((max_seq_len + 63) / 64, num_seqs);
    hipLaunchKernelGGL(head_sum_columns, grid, dim3(64 * kColWaves), 0, stream, scores,
                       score_stride, seq_lens, num_heads, max_seq_len, accumulate, out_max,
                       out_mean, out_seq_stride);
    return hipGetLastError();
  }
  const int n_blk_max = (max_seq_len + block_size - 1) / block_size;
  const long long total = (long long)(head_sum ? num_seqs : num_seqs * num_heads) * n_blk_max;
  const dim3 grid((unsigned)((total + kThreads - 1) / kThreads));
  hipLaunchKernelGGL(block_agg_generic, grid, dim3(kThreads), 0, stream, scores, score_stride,
                     seq_lens, num_seqs, num_heads, n_blk_max, block_size, head_sum, accumulate,
                     out_max, out_mean, out_stride, out_seq_stride);
  return hipGetLastError();
}

}  // namespace kvsel
