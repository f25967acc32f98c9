// Internal launch interface between the C ABI (kvsel_api.cpp) and the HIP
// kernels.  All pointers are device pointers; all sizes were validated by the
// caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvsel.h"

namespace kvsel {

// Split-K decode geometry shared by the launcher and the workspace query.
struct DecodePlan {
  int chunk;      // keys per split-K chunk (multiple of 64)
  int n_chunks;   // ceil(max_seq_len / chunk)
  int gt;         // query heads handled per workgroup (power of two <= 8)
  int hgroups;    // G / gt
  size_t part_o_bytes, part_ml_bytes, lse_bytes, scratch_bytes, sync_bytes, total_bytes;
};

DecodePlan plan_decode(int num_seqs, int num_kv_heads, int num_q_heads, int head_dim,
                       int max_seq_len, bool need_scratch);

struct DecodeArgs {
  const void* k_pages;
  const void* v_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const void* q;
  int num_seqs, num_kv_heads, num_q_heads, head_dim, page_size, max_pages, max_seq_len;
  bool bf16;
  float scale;
  float* out;
  float* lse;
  float* probs;
  int64_t probs_stride;
  bool emit_logits;
  float* cum;
  int64_t cum_stride;
  float decay;
  void* workspace;
  uint32_t epoch;      // unique per call (never 0): tags the row arrival words
  unsigned long long wait_ticks;  // bound of the in-kernel normalisation's wait (wall-clock ticks)
  // Optional block aggregates of the updated cum (blk_bs > 0, cum required).
  int blk_bs;
  float* blk_max;
  float* blk_mean;
  int64_t blk_head_stride, blk_seq_stride;
};

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream);

hipError_t launch_accumulate(const float* probs, int64_t probs_stride, const int32_t* seq_lens,
                             int num_seqs, int num_q_heads, int num_kv_heads, int max_seq_len,
                             float decay, float* cum, int64_t cum_stride, hipStream_t stream);

hipError_t launch_block_aggregate(const float* scores, int64_t score_stride,
                                  const int32_t* seq_lens, int num_seqs, int num_heads,
                                  int max_seq_len, int block_size, bool head_sum, bool accumulate,
                                  float* out_max, float* out_mean, int64_t out_stride,
                                  int64_t out_seq_stride, hipStream_t stream);  // <= 0: packed rows

hipError_t launch_accumulate_ex(const float* probs, int64_t probs_stride, const int32_t* seq_lens, int num_seqs,
                                int num_q_heads, int num_kv_heads, int max_seq_len, int mode, float decay,
                                int window, int step, float* ring, float* cum, int64_t cum_stride,
                                hipStream_t stream);
hipError_t launch_block_variant(const float* scores, int64_t score_stride, const int32_t* seq_lens, int num_seqs,
                                int num_heads, int max_seq_len, int block_size, int mode, float param, float* out,
                                int64_t out_stride, hipStream_t stream);
hipError_t launch_select_threshold(const float* scores, int64_t stride, const int32_t* lengths, int rows,
                                   float threshold, int32_t* out_idx, int64_t out_stride, int32_t* out_count,
                                   hipStream_t stream);

hipError_t launch_union_keep(const int32_t* idx, int64_t idx_stride, const int32_t* counts, int num_seqs,
                             int num_q_heads, int num_kv_heads, int max_len, int32_t* out, int64_t out_stride,
                             int32_t* out_count, hipStream_t stream);

hipError_t launch_indexer_fp8(const void* k_pages, const int32_t* block_table, const int32_t* seq_lens,
                              const void* q, int num_seqs, int num_kv_heads, int num_q_heads, int head_dim,
                              int page_size, int max_pages, int max_seq_len, float scale, float* scores,
                              int64_t stride, hipStream_t stream);

hipError_t launch_block_update(const int32_t* idx, int64_t idx_stride, const int32_t* counts, int rows,
                               int max_count, const float* values, int64_t values_stride, int block_size,
                               int step, float decay, kvsel_block_meta* meta, int64_t meta_stride, hipStream_t stream);

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* out, hipStream_t stream);

size_t select_workspace_bytes(int rows, int max_len, int mode);

// Indexer top-k: the keep sets select_keep (sinks 0, window 0, budget topk)
// would pick from the bf16 indexer's logits, without storing the logits.
struct IndexerTopkArgs {
  const void* k_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const void* q;
  int num_seqs, num_kv_heads, num_q_heads, head_dim, page_size, max_pages, max_seq_len;
  float scale;
  int topk;
  int32_t* keep;
  int64_t keep_stride;
  int32_t* counts;
  void* workspace;
  bool fp8;   // keys and queries in FP8 E4M3 (else bf16)
};
size_t indexer_topk_workspace_bytes(int num_seqs, int num_q_heads, int max_seq_len, int topk);
hipError_t launch_indexer_topk(const IndexerTopkArgs& a, hipStream_t stream);

hipError_t launch_select(const float* scores, int64_t stride, const int32_t* lengths, int rows,
                         int max_len, int sinks, int window, const int32_t* budgets,
                         int max_budget, int mode, int global_budget, int32_t* out_idx,
                         int64_t out_stride, int32_t* out_count, void* workspace,
                         hipStream_t stream);
// Whether launch_select (ROWS mode) splits these rows over workgroups; when it
// does not, every row is selected by the one-workgroup algorithm of
// row_select.hpp, which a caller may then run inside its own kernel.
bool select_rows_split(int rows, int max_len, int max_budget);

struct SparseArgs {
  const void* k_pages;
  const void* v_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const void* q;
  const int32_t* indices;
  int64_t idx_stride;
  const int32_t* counts;
  int num_seqs, num_kv_heads, num_q_heads, head_dim, page_size, max_pages, idx_heads, max_count;
  bool bf16;
  float scale;
  float* out;
  float* probs;
  void* workspace;
  // Listed logits left raw in `probs` (no normalisation pass), with each
  // (sequence, query head)'s log-sum-exp also written to lse_out (or null).
  bool raw_logits;
  float* lse_out;
  // Only the split-K partial pass runs: the caller combines the partials
  // (sparse_partials) itself; out, lse_out and probs normalisation are its own.
  bool partials_only;
  // Each set also holds the current token, position seq_lens[b] - 1, as an
  // entry after its `count` listed ones (when count < max_count), not yet
  // written to `indices`.
  bool append_current;
};

size_t sparse_workspace_bytes(int num_seqs, int num_q_heads, int head_dim, int max_count);
hipError_t launch_sparse(const SparseArgs& a, hipStream_t stream);

// Where launch_sparse leaves its split-K partials in a.workspace: for
// (sequence, query head) bh and chunk c < ceil(count / slice), the chunk's
// (max logit, sum of exp(logit - max)) at part_ml[bh * n_chunks + c] and its
// unnormalised output sum_j exp(s_j - max) v_j at part_o[(bh * n_chunks + c) * D];
// chunk c covers listed entries [c * slice, (c + 1) * slice).
struct SparsePartials {
  float* part_o;
  float2* part_ml;
  int n_chunks, slice;
};
SparsePartials sparse_partials(const SparseArgs& a);

struct SnapkvArgs {
  const void* k_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const void* q_win;
  int num_seqs, num_kv_heads, num_q_heads, head_dim, page_size, max_pages, max_seq_len;
  int window, pool_kernel;
  bool group_sum;
  float scale;
  float* votes;
  int64_t votes_stride;
  void* workspace;
};

size_t snapkv_workspace_bytes(int num_seqs, int num_kv_heads, int num_q_heads, int window, int max_seq_len);
hipError_t launch_snapkv(const SnapkvArgs& a, hipStream_t stream);

// Quest page-bound selection: the paged cache, the queries' shape.
struct QuestArgs {
  const void* k_pages;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int num_seqs, num_kv_heads, num_q_heads, head_dim, page_size, max_pages, max_seq_len;
  bool bf16;
};

hipError_t launch_quest_summary(const QuestArgs& a, void* summary, int first_page, hipStream_t stream);
size_t quest_workspace_bytes(int num_seqs, int num_q_heads, int page_size, int max_seq_len, int budget_pages);
hipError_t launch_quest_select(const QuestArgs& a, const void* summary, const void* q, int budget_pages,
                               const int32_t* query_pos, float* bounds, int64_t bounds_stride, int32_t* out_idx,
                               int64_t out_stride, int32_t* out_count, void* workspace, hipStream_t stream);

// H2O decode step with per-step eviction over per-KV-head slot lists.
struct H2oArgs {
  SparseArgs sp;             // the paged cache, q, out; indices/counts = the slot lists
  int32_t* slots;            // [B][H_kv][slot_stride] ascending positions
  float* slot_cum;           // [B][H_kv][slot_stride]
  int32_t* slot_count;       // [B][H_kv]
  int64_t slot_stride;
  int sinks, window, budget;
  const int32_t* budgets;    // [B][H_kv] per-list budgets (<= budget), or null
  float decay;
};

size_t h2o_workspace_bytes(int num_seqs, int num_kv_heads, int num_q_heads, int head_dim, int64_t slot_stride,
                           int sinks, int window, int budget);
hipError_t launch_h2o_step(const H2oArgs& a, hipStream_t stream);

}  // namespace kvsel
