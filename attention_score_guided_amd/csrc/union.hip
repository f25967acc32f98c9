// Union of the index sets of a GQA group ([EVICT] "KV-cache eviction
// strategies", §4.3 SnapKV under GQA: every query head picks its own top-k
// positions, and the KV head keeps the union of its group's picks, so a
// position any head voted for keeps its K/V for the whole group).
//
// union_keep_kernel: one workgroup per (sequence, KV head).  The positions of
// the group's G lists set bits of a bitmap of the row in LDS (integer
// atomics: order-free, exact); a block scan over the words' popcounts then
// writes the set positions in ascending order.
#include "device_common.hpp"
#include "kvsel_internal.hpp"

namespace kvsel {

namespace {

constexpr int kUThreads = 1024;
constexpr int kUMaxWords = 32768;   // bitmap of up to 2^20 positions (128 KB of LDS)

__global__ __launch_bounds__(kUThreads) void union_keep_kernel(
    const int32_t* __restrict__ idx, int64_t idx_stride, const int32_t* __restrict__ counts, int group,
    int num_kv_heads, int max_len, int32_t* __restrict__ out, int64_t out_stride, int32_t* __restrict__ out_count) {
  extern __shared__ uint32_t bits[];            // [n_words]
  __shared__ int wsum[kUThreads / kWave];
  const int row = blockIdx.x;                   // b * num_kv_heads + kvh
  const int b = row / num_kv_heads, kvh = row % num_kv_heads;
  const int n_words = (max_len + 31) / 32;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  for (int w = tid; w < n_words; w += kUThreads) bits[w] = 0u;
  __syncthreads();
  for (int g = 0; g < group; ++g) {
    const size_t set = (size_t)b * num_kv_heads * group + (size_t)kvh * group + g;
    const int n = counts[set];
    const int32_t* list = idx + set * idx_stride;
    for (int i = tid; i < n; i += kUThreads) {
      const int j = list[i];
      if (j >= 0 && j < max_len) atomicOr(&bits[j >> 5], 1u << (j & 31));
    }
  }
  __syncthreads();
  // each thread owns a contiguous run of words; exclusive scan of the runs'
  // popcounts gives each run's first output slot
  const int per = (n_words + kUThreads - 1) / kUThreads;
  const int w0 = tid * per, w1 = min(n_words, w0 + per);
  int mine = 0;
  for (int w = w0; w < w1; ++w) mine += __popc(bits[w]);
  int incl = mine;
#pragma unroll
  for (int off = 1; off < kWave; off *= 2) {
    const int t = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += t;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < kUThreads / kWave; ++w) {
    before += w < wave ? wsum[w] : 0;
    total += wsum[w];
  }
  int pos = before + incl - mine;
  int32_t* o = out + (size_t)row * out_stride;
  for (int w = w0; w < w1; ++w) {
    uint32_t m = bits[w];
    while (m) {
      const int bit = __ffs(m) - 1;
      o[pos++] = w * 32 + bit;
      m &= m - 1;
    }
  }
  if (tid == 0) out_count[row] = total;
}

}  // namespace

hipError_t launch_union_keep(const int32_t* idx, int64_t idx_stride, const int32_t* counts, int num_seqs,
                             int num_q_heads, int num_kv_heads, int max_len, int32_t* out, int64_t out_stride,
                             int32_t* out_count, hipStream_t stream) {
  const int n_words = (max_len + 31) / 32;
  if (n_words > kUMaxWords) return hipErrorInvalidValue;
  const size_t lds = (size_t)n_words * sizeof(uint32_t);
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&union_keep_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(union_keep_kernel, dim3((unsigned)(num_seqs * num_kv_heads)), dim3(kUThreads),
                     lds, stream, idx, idx_stride, counts,
                     num_q_heads / num_kv_heads, num_kv_heads, max_len, out, out_stride, out_count);
  return hipGetLastError();
}

}  // namespace kvsel
