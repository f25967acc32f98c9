// Score-aggregation variants the pages leave open as design choices.
//
// Across decode steps ([OFFLOAD] "Sparse attention x KV-cache offloading",
// §2.1: sliding-window average, exponential decay, max pooling):
//   accumulate_max_kernel     cum = max(decay * cum, g)
//   accumulate_window_kernel  ring[step % W] = g, cum = (1/W) sum of the ring
// where g is the group sum of one step's probabilities per KV head.
// Token -> block ([OFFLOAD] §3.1 top-p%; [EVICT] §5.1 ranking blocks by their
// share of important tokens, and evicting only all-cold blocks):
//   block_variant_kernel      top-p% mean | fraction >= threshold | all-cold flag
//   (block_variant_lanes: the same for power-of-two blocks of 4..64, one lane per position)
// Across requests ([OFFLOAD] §3.2, absolute-threshold normalisation):
//   select_threshold_kernel   positions with score >= threshold, ascending
// Per-block metadata ([OFFLOAD] §5.1, score accumulator + last-update stamp):
//   block_update_kernel       lazy-decayed score and stamp of the blocks a step selected
// All are HBM-bound streaming passes with one writer per output element.
#include "device_common.hpp"
#include "kvsel_internal.hpp"

namespace kvsel {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float group_prob_sum(const float* pr, int64_t stride, int G, int j) {
  float acc = 0.f;
  for (int g = 0; g < G; ++g) acc += pr[(size_t)g * stride + j];
  return acc;
}

__global__ __launch_bounds__(kThreads) void accumulate_max_kernel(
    const float* __restrict__ probs, int64_t probs_stride, const int32_t* __restrict__ seq_lens, int num_q_heads,
    int num_kv_heads, float decay, float* __restrict__ cum, int64_t cum_stride) {
  const int b = blockIdx.z, c = blockIdx.y;
  const int L = seq_lens[b];
  const int j = blockIdx.x * kThreads + threadIdx.x;
  if (j >= L) return;
  const int G = num_q_heads / num_kv_heads;
  const float g = group_prob_sum(probs + ((size_t)b * num_q_heads + (size_t)c * G) * probs_stride, probs_stride, G, j);
  float* cp = cum + ((size_t)b * num_kv_heads + c) * cum_stride + j;
  *cp = fmaxf(decay * *cp, g);
}

// ring [W][B][H_kv][cum_stride]: slot `slot` receives this step's g, and cum
// the mean of the W slots (summed in slot order: the result does not depend
// on which slot is the newest).
__global__ __launch_bounds__(kThreads) void accumulate_window_kernel(
    const float* __restrict__ probs, int64_t probs_stride, const int32_t* __restrict__ seq_lens, int num_q_heads,
    int num_kv_heads, int num_seqs, int window, int slot, float* __restrict__ ring, float* __restrict__ cum,
    int64_t cum_stride) {
  const int b = blockIdx.z, c = blockIdx.y;
  const int L = seq_lens[b];
  const int j = blockIdx.x * kThreads + threadIdx.x;
  if (j >= L) return;
  const int G = num_q_heads / num_kv_heads;
  const float g = group_prob_sum(probs + ((size_t)b * num_q_heads + (size_t)c * G) * probs_stride, probs_stride, G, j);
  const size_t row = (size_t)b * num_kv_heads + c;
  const size_t plane = (size_t)num_seqs * num_kv_heads * cum_stride;
  float s = 0.f;
  for (int w = 0; w < window; ++w) {
    float* r = ring + w * plane + row * cum_stride + j;
    float v = *r;
    if (w == slot) {
      v = g;
      *r = g;
    }
    s += v;
  }
  cum[row * cum_stride + j] = s / (float)window;
}

// One wave per block of <= 256 positions: its valid scores in LDS; the
// top-p% mean ranks each element by counting the elements that beat it
// (greater, or equal at a lower position), so the m largest are exact and the
// order of equal scores cannot change the sum's terms.
constexpr int kVarWaves = kThreads / kWave;
constexpr int kVarMaxBlock = 256;

__global__ __launch_bounds__(kThreads) void block_variant_kernel(
    const float* __restrict__ scores, int64_t score_stride, const int32_t* __restrict__ seq_lens, int num_heads,
    int block_size, int mode, float param, float* __restrict__ out, int64_t out_stride) {
  __shared__ float v_lds[kVarWaves][kVarMaxBlock];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int b = blockIdx.z, h = blockIdx.y;
  const int L = seq_lens[b];
  const int blk = blockIdx.x * kVarWaves + wave;
  const int start = blk * block_size;
  if (start >= L) return;
  const int n = min(block_size, L - start);
  const float* row = scores + ((size_t)b * num_heads + h) * score_stride + start;
  float* vs = v_lds[wave];
  for (int i = lane; i < n; i += kWave) vs[i] = row[i];
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // the wave's LDS writes before its reads
  __builtin_amdgcn_wave_barrier();
  float res;
  if (mode == 0) {                       // mean of the m = ceil(p * n) largest
    const int m = max(1, min(n, (int)ceilf(param * (float)n)));
    float part = 0.f;
    for (int i = lane; i < n; i += kWave) {
      const float x = vs[i];
      int beat = 0;
      for (int t = 0; t < n; ++t) {
        const float y = vs[t];
        beat += (y > x || (y == x && t < i)) ? 1 : 0;
      }
      if (beat < m) part += x;
    }
    res = wave_sum(part) / (float)m;
  } else {
    int cnt = 0;                          // elements >= threshold
    for (int i = lane; i < n; i += kWave) cnt += vs[i] >= param ? 1 : 0;
    for (int off = kWave / 2; off > 0; off /= 2) cnt += __shfl_xor(cnt, off, kWave);
    res = mode == 1 ? (float)cnt / (float)n : (cnt == 0 ? 1.f : 0.f);
  }
  if (lane == 0) out[((size_t)b * num_heads + h) * out_stride + blk] = res;
}

// Power-of-two blocks of BS <= 64 positions: BS consecutive lanes hold one
// block, one position each (consecutive lanes read consecutive positions);
// the rank of a score counts the lanes of its block that beat it, by
// shuffles; the sums are group reductions.
template <int BS>
__global__ __launch_bounds__(kThreads) void block_variant_lanes(
    const float* __restrict__ scores, int64_t score_stride, const int32_t* __restrict__ seq_lens, int num_heads,
    int mode, float param, float* __restrict__ out, int64_t out_stride) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int L = seq_lens[b];
  const int lane = threadIdx.x % kWave;
  const int blk = blockIdx.x * (kThreads / BS) + threadIdx.x / BS;
  const int i = threadIdx.x % BS;
  const int start = blk * BS;
  if (blockIdx.x * (kThreads / BS) * BS >= L) return;   // the whole workgroup lies past the row
  const int n = start < L ? min(BS, L - start) : 0;
  const float* row = scores + ((size_t)b * num_heads + h) * score_stride;
  const float x = i < n ? row[start + i] : 0.f;
  float part;
  if (mode == 0) {
    const int m = max(1, min(n, (int)ceilf(param * (float)n)));
    int beat = 0;
    const int g0 = lane & ~(BS - 1);
#pragma unroll
    for (int t = 0; t < BS; ++t) {
      const float y = __shfl(x, g0 + t, kWave);
      beat += (t < n && (y > x || (y == x && t < i))) ? 1 : 0;
    }
    part = (i < n && beat < m) ? x : 0.f;
    part = group_sum<BS>(part) / (float)max(m, 1);
  } else {
    part = (i < n && x >= param) ? 1.f : 0.f;
    part = group_sum<BS>(part);                 // exact: small integers
    part = mode == 1 ? part / (float)max(n, 1) : (part == 0.f ? 1.f : 0.f);
  }
  if (i == 0 && n > 0) out[((size_t)b * num_heads + h) * out_stride + blk] = part;
}

// One workgroup per row: the positions with score >= threshold, ascending,
// by a block-wide scan over chunks of kThreads positions.
__global__ __launch_bounds__(kThreads) void select_threshold_kernel(
    const float* __restrict__ scores, int64_t stride, const int32_t* __restrict__ lengths, float threshold,
    int32_t* __restrict__ out_idx, int64_t out_stride, int32_t* __restrict__ out_count) {
  __shared__ int wsum[kThreads / kWave];
  const int r = blockIdx.x;
  const int n = lengths[r];
  const float* row = scores + (size_t)r * stride;
  int32_t* out = out_idx + (size_t)r * out_stride;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  int base = 0;
  for (int j0 = 0; j0 < n; j0 += kThreads) {
    const int j = j0 + tid;
    const int keep = (j < n && row[j] >= threshold) ? 1 : 0;
    // inclusive scan within the wave, then across the waves
    int incl = keep;
#pragma unroll
    for (int off = 1; off < kWave; off *= 2) {
      const int t = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += t;
    }
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) {
      before += w < wave ? wsum[w] : 0;
      total += wsum[w];
    }
    if (keep) out[base + before + incl - 1] = j;
    base += total;
    __syncthreads();
  }
  if (tid == 0) out_count[r] = base;
}

// Per-block metadata update from one step's selection ([OFFLOAD] §5.1: a
// float score accumulator and an int32 last-update stamp per block; each
// step walks the selected blocks).  One thread per list entry (grid: entry
// chunks x rows); the listed positions are ascending, so the positions of a
// block are consecutive among the row's valid entries: the first of them (its
// head) sums them all and is the block's only writer.  score = score *
// decay^(step - stamp) + sum (the stamp makes the decay lazy: untouched
// blocks are not written), stamp = step.  A workgroup stages its entries and
// the next kBUTail ones in LDS, so heads sum from LDS; a block reaching past
// them (long blocks, padding runs) continues from global memory.
constexpr int kBUTail = 64;

// kPow2: block_of (position -> block index) is a shift, for power-of-two
// block sizes (the usual 16, 32 and 64); otherwise it is a division.
template <bool kPow2>
__global__ __launch_bounds__(kThreads) void block_update_kernel(
    const int32_t* __restrict__ idx, int64_t idx_stride, const int32_t* __restrict__ counts, int max_count,
    const float* __restrict__ values, int64_t values_stride, int block_size, int bs_shift, int step, float decay,
    kvsel_block_meta* __restrict__ meta, int64_t meta_stride) {
  __shared__ int32_t sidx[kThreads + kBUTail];
  __shared__ float sval[kThreads + kBUTail];
  auto block_of = [&](int pos) { return kPow2 ? pos >> bs_shift : pos / block_size; };
  const int r = blockIdx.y;
  const int32_t* li = idx + (size_t)r * idx_stride;
  const float* lv = values ? values + (size_t)r * values_stride : nullptr;
  const int i0 = blockIdx.x * kThreads;
  const int i = i0 + threadIdx.x;
  // The count and the own entry load together, and the block's record loads
  // with the staging loads: two dependent memory levels before the store.
  const int n = counts[r];
  const int j = i < max_count ? li[i] : -1;                 // idx_stride >= max_count
  const bool live = i < n && j >= 0;
  const int blk = live ? block_of(j) : 0;
  kvsel_block_meta* m = meta + (size_t)r * meta_stride + blk;
  kvsel_block_meta old{0.f, 0};
  if (live) old = *m;                                       // one 8-byte load
  const int lim = min(n, i0 + kThreads + kBUTail);          // LDS holds entries [i0, lim)
  for (int t = threadIdx.x; t < kThreads + kBUTail; t += kThreads) {
    if (i0 + t < lim) {
      sidx[t] = li[i0 + t];
      sval[t] = lv ? lv[i0 + t] : 1.f;
    }
  }
  __syncthreads();
  if (!live) return;
  int k = i - 1;                                            // previous valid entry
  int jk = -1;
  for (; k >= 0; --k) {
    jk = k >= i0 ? sidx[k - i0] : li[k];
    if (jk >= 0) break;
  }
  if (k >= 0 && block_of(jk) == blk) return;             // not the block's first entry
  // The block's entries, summed in list order: eight LDS entries per round
  // (independent reads, one latency per round), then one at a time past the
  // staged range.
  float sum = 0.f;
  int t = i;
  bool done = false;
  for (; !done && t + 8 <= lim; t += 8) {
    int jj[8];
    float vv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      jj[u] = sidx[t + u - i0];
      vv[u] = sval[t + u - i0];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (!done && jj[u] >= 0) {
        if (block_of(jj[u]) != blk) done = true;
        else sum += vv[u];
      }
    }
  }
  for (; !done && t < n; ++t) {
    const bool in_lds = t < lim;
    const int jt = in_lds ? sidx[t - i0] : li[t];
    if (jt < 0) continue;
    if (block_of(jt) != blk) break;
    sum += in_lds ? sval[t - i0] : (lv ? lv[t] : 1.f);
  }
  const float keep = decay == 1.f ? 1.f : powf(decay, (float)(step - old.stamp));
  *m = kvsel_block_meta{fmaf(keep, old.score, sum), step};  // one 8-byte store
}

}  // namespace

hipError_t launch_block_update(const int32_t* idx, int64_t idx_stride, const int32_t* counts, int rows,
                               int max_count, const float* values, int64_t values_stride, int block_size,
                               int step, float decay, kvsel_block_meta* meta, int64_t meta_stride, hipStream_t stream) {
  if (max_count == 0) return hipSuccess;
  const dim3 grid((max_count + kThreads - 1) / kThreads, rows);
  if ((block_size & (block_size - 1)) == 0) {
    const int shift = __builtin_ctz((unsigned)block_size);
    hipLaunchKernelGGL(block_update_kernel<true>, grid, dim3(kThreads), 0, stream, idx, idx_stride, counts,
                       max_count, values, values_stride, block_size, shift, step, decay, meta, meta_stride);
  } else {
    hipLaunchKernelGGL(block_update_kernel<false>, grid, dim3(kThreads), 0, stream, idx, idx_stride, counts,
                       max_count, values, values_stride, block_size, 0, step, decay, meta, meta_stride);
  }
  return hipGetLastError();
}

hipError_t launch_accumulate_ex(const float* probs, int64_t probs_stride, const int32_t* seq_lens, int num_seqs,
                                int num_q_heads, int num_kv_heads, int max_seq_len, int mode, float decay,
                                int window, int step, float* ring, float* cum, int64_t cum_stride,
                                hipStream_t stream) {
  const dim3 grid((max_seq_len + kThreads - 1) / kThreads, num_kv_heads, num_seqs);
  if (mode == 0)
    return launch_accumulate(probs, probs_stride, seq_lens, num_seqs, num_q_heads, num_kv_heads, max_seq_len, decay,
                             cum, cum_stride, stream);
  if (mode == 1)
    hipLaunchKernelGGL(accumulate_max_kernel, grid, dim3(kThreads), 0, stream, probs, probs_stride, seq_lens,
                       num_q_heads, num_kv_heads, decay, cum, cum_stride);
  else
    hipLaunchKernelGGL(accumulate_window_kernel, grid, dim3(kThreads), 0, stream, probs, probs_stride, seq_lens,
                       num_q_heads, num_kv_heads, num_seqs, window, step % window, ring, cum, cum_stride);
  return hipGetLastError();
}

hipError_t launch_block_variant(const float* scores, int64_t score_stride, const int32_t* seq_lens, int num_seqs,
                                int num_heads, int max_seq_len, int block_size, int mode, float param, float* out,
                                int64_t out_stride, hipStream_t stream) {
  const int n_blk = (max_seq_len + block_size - 1) / block_size;
#define KVSEL_LANES(BS)                                                                                        \
  case BS:                                                                                                     \
    hipLaunchKernelGGL(block_variant_lanes<BS>, dim3((n_blk + kThreads / BS - 1) / (kThreads / BS), num_heads,  \
                       num_seqs), dim3(kThreads), 0, stream, scores, score_stride, seq_lens, num_heads, mode,   \
                       param, out, out_stride);                                                                \
    return hipGetLastError();
  switch (block_size) {
    KVSEL_LANES(4)
    KVSEL_LANES(8)
    KVSEL_LANES(16)
    KVSEL_LANES(32)
    KVSEL_LANES(64)
    default: break;
  }
#undef KVSEL_LANES
  const dim3 grid((n_blk + kVarWaves - 1) / kVarWaves, num_heads, num_seqs);
  hipLaunchKernelGGL(block_variant_kernel, grid, dim3(kThreads), 0, stream, scores, score_stride, seq_lens, num_heads,
                     block_size, mode, param, out, out_stride);
  return hipGetLastError();
}

hipError_t launch_select_threshold(const float* scores, int64_t stride, const int32_t* lengths, int rows,
                                   float threshold, int32_t* out_idx, int64_t out_stride, int32_t* out_count,
                                   hipStream_t stream) {
  hipLaunchKernelGGL(select_threshold_kernel, dim3(rows), dim3(kThreads), 0, stream, scores, stride, lengths,
                     threshold, out_idx, out_stride, out_count);
  return hipGetLastError();
}

}  // namespace kvsel
