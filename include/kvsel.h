/*
 * kvsel.h -- C ABI of the score-guided KV selection library (libkvsel.so).
 *
 * The library computes, on one AMD Instinct MI355X (gfx950), the hot path of
 * attention-score-guided KV-cache management:
 *   decode attention over a paged KV cache that also emits every key's softmax
 *   probability -> H2O cumulative scores per KV head -> token-to-block
 *   aggregation -> keep sets (sinks + heavy hitters + recent window), plus the
 *   SnapKV observation-window vote and sparse attention over an index set.
 *
 * Sources, cited by title and section:
 *   [OFFLOAD] "Sparse attention x KV-cache offloading: eight questions a
 *             cross-layer design must answer"
 *   [EVICT]   "KV-cache eviction strategies: from attention sinks to H2O and
 *             SnapKV"
 *   [LONGCTX] "Long context, KV eviction and sparse attention" (AI-infra
 *             handbook, serving chapter)
 *
 * Conventions (every call):
 *   - Tensor pointers are DEVICE pointers, allocated and owned by the caller.
 *     The library allocates nothing and frees nothing.  Its only state is a
 *     per-device architecture check, a per-call counter that tags the decode
 *     pass's synchronisation words, and the wait bound below.  Scratch space
 *     is passed in as `workspace` (device memory, size from the matching
 *     *_workspace_bytes); two calls must not share a workspace concurrently.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and returns a kvsel_status.  Nothing is synchronised inside.
 *   - Host-visible arguments are validated before any HIP call; on error the
 *     call returns KVSEL_ERR_INVALID / _UNSUPPORTED / _WORKSPACE, launches
 *     nothing, and kvsel_last_error() (thread-local) says why.
 *   - Device-resident values (seq_lens, block tables, indices, budgets) are
 *     preconditions and are not read by the host; each call lists its own
 *     under "Preconditions".  In general: lengths lie in [1, max_seq_len],
 *     block-table entries name pages of the pool, index lists hold distinct
 *     positions < the row length, counts and budgets stay within the
 *     host-known bounds passed beside them, scores are finite or -inf (no
 *     NaN).  A violation gives undefined results and may make a kernel read
 *     or write outside the caller's buffers (a page id outside the pool is
 *     dereferenced as given); only the counts of kvsel_sparse_attn are
 *     clamped, because that costs nothing.
 *   - Results are bitwise reproducible for identical inputs (no float
 *     atomics; every output element has exactly one writer).
 *   - Strides are in elements.  Row-major layouts are spelled out per call.
 *   - Query head h reads KV head h / G with G = num_q_heads / num_kv_heads
 *     (grouped-query attention, repeat-interleaved KV heads as in [LONGCTX]
 *     "sparse attention" experiment).
 */
#ifndef KVSEL_H
#define KVSEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVSEL_OK = 0,
  KVSEL_ERR_INVALID = -1,     /* an argument is out of its documented range  */
  KVSEL_ERR_UNSUPPORTED = -2, /* valid, but a shape/dtype the library does not run */
  KVSEL_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required  */
  KVSEL_ERR_HIP = -4          /* a HIP runtime call or launch failed         */
} kvsel_status;

typedef enum { KVSEL_F32 = 0, KVSEL_BF16 = 1, KVSEL_FP8_E4M3 = 2 /* kvsel_indexer_scores_fp8 only */ } kvsel_dtype;
typedef enum { KVSEL_EMIT_PROBS = 0, KVSEL_EMIT_LOGITS = 1 } kvsel_emit;
typedef enum { KVSEL_REDUCE_NONE = 0, KVSEL_REDUCE_SUM = 1 } kvsel_reduce;
typedef enum { KVSEL_SELECT_ROWS = 0, KVSEL_SELECT_GLOBAL_PERCENTILE = 1 } kvsel_select_mode;

/* One layer's paged KV cache ([EVICT] prerequisites: PagedAttention block
 * table).  Position j of sequence b lives in page block_table[b][j / page_size]
 * at row j % page_size.  Each (page, kv head) tile of page_size x head_dim
 * elements is contiguous. */
typedef struct {
  const void* k_pages;        /* [num_pages][num_kv_heads][page_size][head_dim] */
  const void* v_pages;        /* same layout; NULL when no output is wanted     */
  const int32_t* block_table; /* [num_seqs][max_pages_per_seq] page ids          */
  const int32_t* seq_lens;    /* [num_seqs]; 1 <= L_b <= max_seq_len             */
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t head_dim;           /* 64 or 128                                       */
  int32_t page_size;          /* power of two in [16, 256]                       */
  int32_t max_pages_per_seq;  /* >= ceil(max_seq_len / page_size)                */
  int32_t max_seq_len;        /* host-known bound on every L_b (grid sizing)     */
  int32_t dtype;              /* kvsel_dtype of k_pages, v_pages and queries     */
} kvsel_paged_kv;

/* ------------------------------------------------------------------------
 * Decode attention that emits per-key scores, with fused H2O accumulation.
 *
 * [OFFLOAD] §1.1 and §1.3: attention computes each key's importance every
 * decode step and engines discard it; [EVICT] §4.2 (H2O): each step's
 * attention weights are added to a per-position cumulative score.
 *
 * For sequence b, query head h (KV head c = h / G) and every key j < L_b:
 *   s_j = scale * q[b][h] . k[c][j]
 *   probs[b][h][j] = exp(s_j - lse[b][h])        (emit = KVSEL_EMIT_PROBS)
 *   probs[b][h][j] = s_j                         (emit = KVSEL_EMIT_LOGITS)
 *   out[b][h][:]   = sum_j softmax(s)_j v[c][j]
 *   lse[b][h]      = ln sum_j exp(s_j)
 *   cum[b][c][j]   = decay * cum[b][c][j] + sum_{h in group c} probs[b][h][j]
 * The query is the current token; its key/value must already be appended,
 * so the query sees L_b keys including its own.
 *
 *   q      [num_seqs][num_q_heads][head_dim], dtype kv->dtype.
 *   out    [num_seqs][num_q_heads][head_dim] f32, or NULL.  Needs v_pages.
 *   lse    [num_seqs][num_q_heads] f32, or NULL.
 *   probs  [num_seqs][num_q_heads][probs_stride] f32, or NULL; entries at
 *          j >= L_b are left untouched.  probs_stride >= max_seq_len.
 *   cum    [num_seqs][num_kv_heads][cum_stride] f32, read and written, or
 *          NULL.  Needs emit = PROBS.  cum_stride >= max_seq_len.
 *          probs and cum rows that are 16-byte aligned (base aligned, stride
 *          a multiple of 4) take 16-byte stores; other layouts are accepted
 *          and take 4-byte stores (in the bf16 logits-only mode of an
 *          indexer, runs of 16 keys staged through LDS: ~25% slower there).
 *   workspace: >= kvsel_decode_workspace_bytes(kv, num_q_heads,
 *          probs != NULL || cum == NULL) bytes of device memory, 256-byte
 *          aligned, contents ignored.
 * Preconditions: 1 <= seq_lens[b] <= max_seq_len; block_table[b][p] names a
 * page of k_pages (and v_pages) for every p < ceil(L_b / page_size); probs,
 * cum and workspace do not overlap each other or the inputs.
 * Supported: head_dim 64/128; dtype F32/BF16; G a power of two <= 8 or a
 * multiple of 8.  Errors: INVALID (NULL kv/q/k_pages/block_table/seq_lens,
 * dims <= 0, num_q_heads % num_kv_heads != 0, stride < max_seq_len,
 * out != NULL without v_pages, max_pages_per_seq too small), UNSUPPORTED
 * (head_dim, dtype, page_size, G, cum with emit = LOGITS, no gfx950 device),
 * WORKSPACE, HIP.
 * ------------------------------------------------------------------------ */
int kvsel_decode_attn_scores(const kvsel_paged_kv* kv, const void* q, int32_t num_q_heads,
                             float scale, float* out, float* lse, float* probs,
                             int64_t probs_stride, int32_t emit, float* cum, int64_t cum_stride,
                             float decay, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * kvsel_decode_attn_scores without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP-graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The call computes exactly what
 * kvsel_decode_attn_scores computes (same kernels) and allocates nothing
 * (no hipMalloc / hipFree, no allocating library routine).  Its scratch is a
 * static device array of KVSEL_NOALLOC_SCRATCH_BYTES that every device the
 * library runs on holds until the process ends; its device address is looked
 * up once per device, on that device's first call.
 *   Size limit: calls whose workspace (kvsel_decode_workspace_bytes with
 *   probs_given = (probs != NULL || cum == NULL)) exceeds the array return
 *   KVSEL_ERR_WORKSPACE before any HIP call.  The 70B-shape layer (8 x 32K,
 *   64/8 heads, probs given) needs ~9 MB; cum without probs adds
 *   num_seqs * num_q_heads * max_seq_len * 4 bytes.
 *   Sharing: all calls on one device share its array, which keeps the last
 *   call's contents; calls that overlap in time on one device (different
 *   streams or threads) race and give undefined results.  Stream-ordered
 *   calls are safe.
 * Arguments, results and other errors as kvsel_decode_attn_scores.
 * ------------------------------------------------------------------------ */
#define KVSEL_NOALLOC_SCRATCH_BYTES (96u << 20)

int kvsel_decode_attn_scores_noalloc(const kvsel_paged_kv* kv, const void* q, int32_t num_q_heads,
                                     float scale, float* out, float* lse, float* probs,
                                     int64_t probs_stride, int32_t emit, float* cum, int64_t cum_stride,
                                     float decay, void* stream);

/* Workspace bytes for kvsel_decode_attn_scores (0 if the arguments are
 * invalid).  probs_given = 0 adds the logits scratch needed when cum is
 * fused without a caller probs buffer (an upper bound for every call). */
size_t kvsel_decode_workspace_bytes(const kvsel_paged_kv* kv, int32_t num_q_heads,
                                    int32_t probs_given);

/* ------------------------------------------------------------------------
 * Standalone H2O accumulation ([EVICT] §4.2; decay < 1 is the exponential
 * decay aggregation of [OFFLOAD] §2.1):
 *   cum[b][c][j] = decay * cum[b][c][j] + sum_{h: h / G == c} probs[b][h][j],
 * for j < seq_lens[b].  probs [num_seqs][num_q_heads][probs_stride] f32,
 * cum [num_seqs][num_kv_heads][cum_stride] f32 (in place).
 * Preconditions: 1 <= seq_lens[b] <= max_seq_len.  Errors: INVALID.
 * ------------------------------------------------------------------------ */
int kvsel_accumulate(const float* probs, int64_t probs_stride, const int32_t* seq_lens,
                     int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t max_seq_len, float decay, float* cum, int64_t cum_stride,
                     void* stream);

/* ------------------------------------------------------------------------
 * Decode attention with the token-to-block aggregation of the updated
 * cumulative scores in the same pass ([OFFLOAD] §3.1 and §5.1 on top of the
 * call above): identical to kvsel_decode_attn_scores with emit = PROBS and
 * cum != NULL, and in addition, for every (sequence b, KV head h) and block
 * n < ceil(L_b / block_size) of positions [n*block_size, min((n+1)*block_size,
 * L_b)), the max (blk_max) and mean (blk_mean) of the updated cum there,
 * written at blk_*[b * blk_seq_stride + h * blk_head_stride + n].  Other
 * entries are left untouched.  Either output may be NULL (not both).
 * blk_head_stride >= ceil(max_seq_len / block_size) and blk_seq_stride >=
 * num_kv_heads * blk_head_stride; a larger blk_seq_stride lets the blocks of
 * several layers be stacked as extra heads of one array, so one
 * kvsel_block_aggregate call (block_size 1, head_reduce SUM) sums them over
 * heads and layers.  For bf16 caches with G <= 8 and power-of-two block sizes
 * 4..256 the blocks come out of the attention pass itself; otherwise the
 * aggregation runs after it (same results).  Workspace as for
 * kvsel_decode_attn_scores with these probs and cum.
 * Errors: as kvsel_decode_attn_scores, plus INVALID for cum == NULL, both
 * block outputs NULL, block_size <= 0 or strides too small.
 * ------------------------------------------------------------------------ */
int kvsel_decode_attn_scores_agg(const kvsel_paged_kv* kv, const void* q, int32_t num_q_heads,
                                 float scale, float* out, float* lse, float* probs,
                                 int64_t probs_stride, float* cum, int64_t cum_stride, float decay,
                                 int32_t block_size, float* blk_max, float* blk_mean,
                                 int64_t blk_head_stride, int64_t blk_seq_stride, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Token-to-block aggregation ([OFFLOAD] §3.1: max keeps a block holding any
 * key token, mean dilutes it).  Block n of row (b, h) covers positions
 * [n*block_size, min((n+1)*block_size, L_b)); a partial last block aggregates
 * its valid positions only (mean divides by their count).
 *   scores   [num_seqs][num_heads][score_stride] f32.
 *   head_reduce = NONE: out_* [num_seqs][num_heads][out_stride];
 *   head_reduce = SUM:  out_* [num_seqs][out_stride], summed over heads (the
 *                       one accumulator per block of [OFFLOAD] §5.1).
 *   accumulate = 1 adds into out_* (e.g. a sum over layers); 0 overwrites.
 * Blocks n >= ceil(L_b / block_size) are left untouched.  Either output may
 * be NULL (not both).  out_stride >= ceil(max_seq_len / block_size).
 * Preconditions: 1 <= seq_lens[b] <= max_seq_len.
 * Errors: INVALID.
 * ------------------------------------------------------------------------ */
int kvsel_block_aggregate(const float* scores, int64_t score_stride, const int32_t* seq_lens,
                          int32_t num_seqs, int32_t num_heads, int32_t max_seq_len,
                          int32_t block_size, int32_t head_reduce, int32_t accumulate,
                          float* out_max, float* out_mean, int64_t out_stride, void* stream);

/* ------------------------------------------------------------------------
 * Keep-set selection.
 *
 * mode = ROWS ([EVICT] §4.2 H2O; §4.1 StreamingLLM is sinks = 4, window =
 * budget - 4, and the sliding window is sinks = 0, window = budget): for row
 * r of length n = lengths[r] and budget B_r (budgets[r], or max_budget when
 * budgets is NULL):
 *   if B_r >= n every position is kept; otherwise the forced positions
 *   [0, min(sinks, n)) and [max(n - window, 0), n) are kept, plus the
 *   max(0, B_r - |forced|) middle positions with the highest scores (equal
 *   scores: lower position first; -0.0 equals +0.0; NaN is a precondition
 *   violation; -inf ranks lowest).
 * mode = GLOBAL_PERCENTILE ([OFFLOAD] §3.2): every position gets the
 *   percentile (rank + 1) / n of its score within its own row (rank ascending,
 *   equal scores: the lower position ranks higher); the global_budget
 *   positions with the highest percentiles over all rows are kept (ties: lower
 *   row, then lower position).  sinks and window must be 0.  Supported:
 *   max_len <= 8192 and rows * max_len <= 2^20 (else UNSUPPORTED).
 * Output: out_idx[r][0 .. out_count[r]) holds the kept positions ascending;
 *   the rest of the row is left untouched.
 *   scores [rows][stride] f32, lengths [rows] i32 (1 <= n <= max_len),
 *   out_idx [rows][out_stride] i32, out_count [rows] i32.
 *   out_stride >= min(max_len, max(max_budget, sinks + window)) in ROWS mode
 *   (budgets[r] <= max_budget is a precondition) and >= max_len in
 *   GLOBAL_PERCENTILE mode.
 *   Preconditions: 1 <= lengths[r] <= max_len; 0 <= budgets[r] <= max_budget;
 *   scores[r][j] for j < lengths[r] finite or -inf (NaN has no place in the
 *   order).
 *   workspace: >= kvsel_select_workspace_bytes(rows, max_len, mode) bytes
 *   (device memory, any contents; may be 0 bytes).  ROWS mode needs one only
 *   for shapes whose long rows it may split over several workgroups (at most
 *   2048 rows of max_len >= 16384; it splits when also max_budget <=
 *   max_len / 8); the result is the same either way.
 * Errors: INVALID (NULL pointers, rows/max_len <= 0, stride < max_len,
 * negative sinks/window/max_budget/global_budget, out_stride too small,
 * GLOBAL with sinks or window), UNSUPPORTED, WORKSPACE, HIP.
 * ------------------------------------------------------------------------ */
int kvsel_select_keep(const float* scores, int64_t stride, const int32_t* lengths, int32_t rows,
                      int32_t max_len, int32_t sinks, int32_t window, const int32_t* budgets,
                      int32_t max_budget, int32_t mode, int32_t global_budget, int32_t* out_idx,
                      int64_t out_stride, int32_t* out_count, void* workspace,
                      size_t workspace_bytes, void* stream);

size_t kvsel_select_workspace_bytes(int32_t rows, int32_t max_len, int32_t mode);

/* ------------------------------------------------------------------------
 * SnapKV observation-window vote ([EVICT] §4.3, steps 2-4).
 * The `window` queries of each sequence sit at positions L_b - window + i,
 * i < window, and each takes a causal softmax over keys 0 .. L_b - window + i.
 * For prefix keys j < L_b - window:
 *   vote_h[j] = sum_i softmax_i(j)              (sum pooling per query head)
 *   group_reduce = SUM:  g = kv head, votes = sum of the group's vote_h
 *   group_reduce = NONE: g = query head
 *   votes[b][g][j] = max_{|t| <= pool_kernel/2, 0 <= j+t < L_b - window} vote[j+t]
 *   q_win [num_seqs][num_q_heads][window][head_dim] (dtype kv->dtype),
 *   votes [num_seqs][H_kv or H_q][votes_stride] f32; positions
 *   j >= L_b - window are left untouched.  votes_stride >= max_seq_len.
 * Preconditions: window < L_b <= max_seq_len for every sequence; block-table
 * entries as for kvsel_decode_attn_scores.
 *   workspace: >= kvsel_snapkv_workspace_bytes(kv, num_q_heads, window).
 * Errors: INVALID (NULL pointers, window <= 0, window >= max_seq_len, even or
 * non-positive pool_kernel, votes_stride < max_seq_len), UNSUPPORTED (dtype
 * other than BF16, head_dim other than 64/128, window > 64, pool_kernel > 17),
 * WORKSPACE, HIP.
 * ------------------------------------------------------------------------ */
int kvsel_snapkv_vote(const kvsel_paged_kv* kv, const void* q_win, int32_t num_q_heads,
                      int32_t window, int32_t pool_kernel, float scale, int32_t group_reduce,
                      float* votes, int64_t votes_stride, void* workspace,
                      size_t workspace_bytes, void* stream);

size_t kvsel_snapkv_workspace_bytes(const kvsel_paged_kv* kv, int32_t num_q_heads, int32_t window);

/* ------------------------------------------------------------------------
 * Sparse attention over an index set ([LONGCTX] sparse-attention experiment:
 * the softmax runs over the selected keys only; DeepSeek-style indexers pick
 * 2048 keys per query).
 * idx_heads = num_q_heads: one set per query head; idx_heads = num_kv_heads:
 * one set shared by the query heads of a group (G a power of two <= 8).
 *   indices [num_seqs][idx_heads][idx_stride] i32 logical positions < L_b,
 *           distinct; entries < 0 are ignored; only the first counts[b][g]
 *           entries of a row are read.
 *   counts  [num_seqs][idx_heads] i32, 0 <= counts <= max_count <= idx_stride
 *           (a precondition; a larger count is read as max_count, so no
 *           access leaves the index rows or the workspace).
 *   out     [num_seqs][num_q_heads][head_dim] f32 (all zero for an empty set).
 *   probs   [num_seqs][num_q_heads][idx_stride] f32 or NULL: entry i < count
 *           receives the probability of the listed position (0 for an ignored
 *           entry); entries past the count are left untouched.
 *   workspace: >= kvsel_sparse_workspace_bytes(num_seqs, num_q_heads,
 *           head_dim, max_count) bytes of device memory.
 * Preconditions: the non-negative entries of a row are distinct positions
 * < L_b (a repeat would count its key twice in the softmax); L_b and the
 * block table as for kvsel_decode_attn_scores; counts as above.
 * Errors: INVALID, UNSUPPORTED (also max_count > 2^24), WORKSPACE, HIP.
 * ------------------------------------------------------------------------ */
int kvsel_sparse_attn(const kvsel_paged_kv* kv, const void* q, int32_t num_q_heads,
                      const int32_t* indices, int64_t idx_stride, const int32_t* counts,
                      int32_t idx_heads, int32_t max_count, float scale, float* out,
                      float* probs, void* workspace, size_t workspace_bytes, void* stream);

size_t kvsel_sparse_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                    int32_t max_count);

/* ------------------------------------------------------------------------
 * Score-aggregation variants that the pages leave open as design choices.
 *
 * kvsel_accumulate_ex: one step's probabilities folded across decode steps
 * ([OFFLOAD] §2.1: exponential decay, max pooling, sliding-window average).
 * With g[b][c][j] = sum over the query heads of KV head c of probs[b][h][j],
 * for j < L_b:
 *   KVSEL_ACC_SUM (0):         cum = decay * cum + g    (H2O; = kvsel_accumulate)
 *   KVSEL_ACC_MAX (1):         cum = max(decay * cum, g)
 *   KVSEL_ACC_WINDOW_MEAN (2): ring[step % window][b][c][j] = g, then
 *                              cum = (sum of the `window` ring slots) / window
 *                              (slots never written count as 0: the ring must
 *                              start zeroed).
 *   ring  [window][num_seqs][num_kv_heads][cum_stride] f32 (WINDOW_MEAN only).
 * Errors: INVALID (NULL pointers, bad dims, strides, mode, window <= 0 or
 * step < 0 for WINDOW_MEAN), HIP.
 * ------------------------------------------------------------------------ */
typedef enum { KVSEL_ACC_SUM = 0, KVSEL_ACC_MAX = 1, KVSEL_ACC_WINDOW_MEAN = 2 } kvsel_acc_mode;

int kvsel_accumulate_ex(const float* probs, int64_t probs_stride, const int32_t* seq_lens, int32_t num_seqs,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t max_seq_len, int32_t mode,
                        float decay, int32_t window, int32_t step, float* ring, float* cum, int64_t cum_stride,
                        void* stream);

/* kvsel_block_aggregate_ex: one score per block of `block_size` positions
 * (the last block partial: only valid positions count), per (b, h):
 *   KVSEL_BLOCK_TOP_P_MEAN (0): mean of the m = max(1, ceil(param * n)) largest
 *     scores of the block's n valid positions ([OFFLOAD] §3.1 "top-p%", read
 *     as the mean of the block's top p fraction: between max and mean);
 *   KVSEL_BLOCK_FRAC_ABOVE (1): fraction of the n positions with score >= param
 *     ([EVICT] §5.1: rank blocks by their share of important tokens);
 *   KVSEL_BLOCK_ALL_COLD (2): 1 when every position scores < param, else 0
 *     ([EVICT] §5.1: evict only blocks that are cold throughout).
 *   out [num_seqs][num_heads][out_stride] f32, out_stride >= ceil(max_seq_len /
 *   block_size); block_size in [1, 256].
 * Errors: INVALID, UNSUPPORTED (block_size > 256), HIP.
 * ------------------------------------------------------------------------ */
typedef enum { KVSEL_BLOCK_TOP_P_MEAN = 0, KVSEL_BLOCK_FRAC_ABOVE = 1, KVSEL_BLOCK_ALL_COLD = 2 } kvsel_block_mode;

int kvsel_block_aggregate_ex(const float* scores, int64_t score_stride, const int32_t* seq_lens, int32_t num_seqs,
                             int32_t num_heads, int32_t max_seq_len, int32_t block_size, int32_t mode, float param,
                             float* out, int64_t out_stride, void* stream);

/* kvsel_block_update: per-block metadata from one decode step's selection
 * ([OFFLOAD] §5.1: a float score accumulator and an int32 last-update stamp,
 * 8 bytes per block, updated by walking the blocks each step selected).  The
 * two live side by side in one kvsel_block_meta record, so an update touches
 * one cache line per block.  For row r and every block b holding at least one
 * listed position j (j / block_size = b) of idx[r][0 .. counts[r]):
 *   meta[r][b].score = meta[r][b].score * decay^(step - meta[r][b].stamp)
 *                      + sum of values[r][i] over the listed positions i of
 *                        block b (values NULL: 1 each)
 *   meta[r][b].stamp = step
 * Blocks without a listed position are not touched: the stamp makes the decay
 * lazy.  Lists are ascending among their non-negative entries; negative
 * entries are ignored.  meta [rows][meta_stride] records, meta_stride >= max
 * block index + 1 (a precondition); values [rows][values_stride] aligned with
 * idx (e.g. the probabilities that kvsel_sparse_attn emits for the same
 * lists); counts[r] <= max_count (a precondition).
 * Errors: INVALID (NULL pointers, rows <= 0, block_size <= 0, a stride
 * smaller than max_count), UNSUPPORTED (rows > 65535), HIP.
 * ------------------------------------------------------------------------ */
typedef struct {
  float score;
  int32_t stamp;
} kvsel_block_meta;

int kvsel_block_update(const int32_t* idx, int64_t idx_stride, const int32_t* counts, int32_t rows,
                       int32_t max_count, const float* values, int64_t values_stride, int32_t block_size,
                       int32_t step, float decay, kvsel_block_meta* meta, int64_t meta_stride, void* stream);

/* kvsel_select_threshold: absolute-threshold selection across requests
 * ([OFFLOAD] §3.2): per row r, the positions j < lengths[r] with
 * scores[r][j] >= threshold, ascending, and their count.  out_stride >= max_len.
 * Errors: INVALID, HIP.
 * ------------------------------------------------------------------------ */
int kvsel_select_threshold(const float* scores, int64_t stride, const int32_t* lengths, int32_t rows,
                           int32_t max_len, float threshold, int32_t* out_idx, int64_t out_stride,
                           int32_t* out_count, void* stream);

/* ------------------------------------------------------------------------
 * Union of a GQA group's index sets ([EVICT] §4.3, SnapKV under GQA: each
 * query head picks its own positions, the KV head keeps the union).
 *   idx     [num_seqs][num_q_heads][idx_stride] i32 positions (entries < 0 or
 *           >= max_len are ignored; only the first counts[b][h] are read)
 *   counts  [num_seqs][num_q_heads] i32
 *   out     [num_seqs][num_kv_heads][out_stride] i32: the union, ascending,
 *           without repeats; out_count [num_seqs][num_kv_heads].
 *   out_stride >= min(max_len, G * idx_stride); max_len <= 2^20.
 * Errors: INVALID (NULL pointers, bad dims or strides), UNSUPPORTED
 * (max_len > 2^20), HIP.
 * ------------------------------------------------------------------------ */
int kvsel_union_keep(const int32_t* idx, int64_t idx_stride, const int32_t* counts, int32_t num_seqs,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t max_len, int32_t* out,
                     int64_t out_stride, int32_t* out_count, void* stream);

/* ------------------------------------------------------------------------
 * FP8 indexer scores ([LONGCTX] sparse-attention section: a lightweight
 * indexer with few heads scores every token in FP8; the top 2048 per query
 * feed the sparse attention).  kv->dtype must be KVSEL_FP8_E4M3 (OCP E4M3:
 * 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, the
 * all-ones code NaN, max 448); kv->v_pages is not read.
 *   q       [num_seqs][num_q_heads][head_dim] E4M3, 16-byte aligned
 *   scores  [num_seqs][num_q_heads][stride] f32: scale * q . k_j for j < L_b
 *           (query head h reads indexer head h / G), products accumulated in
 *           fp32; entries j >= L_b are left untouched.  stride >= max_seq_len.
 * Errors: INVALID (NULL pointers, stride, dtype not FP8_E4M3, unaligned q or
 * pages), UNSUPPORTED (as the descriptor checks), HIP.
 * ------------------------------------------------------------------------ */
int kvsel_indexer_scores_fp8(const kvsel_paged_kv* kv, const void* q, int32_t num_q_heads, float scale,
                             float* scores, int64_t stride, void* stream);

/* ------------------------------------------------------------------------
 * Indexer top-k ([LONGCTX] "sparse attention" experiment: the indexer scores
 * every cached key of a query and the query attends to its top 2048 keys).
 * For sequence b and query head h (indexer KV head c = h / G), with
 * s_j = scale * q[b][h] . k[c][j] for the L_b cached keys j < L_b:
 *   keep[b * num_q_heads + h][0 .. n)  the positions of the min(topk, L_b)
 *        largest s_j, equal scores resolved toward the lower position,
 *        ascending;  counts[b * num_q_heads + h] = n.
 * The sets are exactly those of kvsel_decode_attn_scores (EMIT_LOGITS, same
 * scale) -- or, for FP8 E4M3 pages, kvsel_indexer_scores_fp8 -- followed by
 * kvsel_select_keep (ROWS mode, sinks 0, window 0, budgets NULL, max_budget
 * topk) on the scores, without the scores being written: long rows compute
 * them where the selection needs them (sampled positions, the pass that
 * stores the keys at or above a sampled lower bound of the cut, and a row's
 * fallback) with the same products in the same order.
 *   kv      bf16 or FP8 E4M3 pages (kv->dtype KVSEL_BF16 or KVSEL_FP8_E4M3),
 *           head_dim 64 or 128; v_pages is not read.
 *   q       [num_seqs][num_q_heads][head_dim] in the pages' format; FP8 q
 *           and pages 16-byte aligned.
 *   keep    [num_seqs * num_q_heads][keep_stride] i32, keep_stride >=
 *           min(topk, max_seq_len); entries past counts are left untouched.
 *   workspace: >= kvsel_indexer_topk_workspace_bytes(kv, num_q_heads, topk)
 *           bytes of device memory, 256-byte aligned, contents ignored.
 * Preconditions as kvsel_decode_attn_scores (1 <= seq_lens[b] <=
 * max_seq_len, block table entries name pages); keep, counts and workspace
 * do not overlap each other or the inputs.
 * Supported: G = num_q_heads / num_kv_heads a power of two <= 8 or 16, 24,
 * 32.  Errors: INVALID (NULL pointers, dims, topk < 1, keep_stride, unaligned
 * FP8 q or pages), UNSUPPORTED (dtype other than BF16 or FP8_E4M3, head_dim,
 * page_size, G, no gfx950 device), WORKSPACE, HIP.
 * ------------------------------------------------------------------------ */
int kvsel_indexer_topk(const kvsel_paged_kv* kv, const void* q, int32_t num_q_heads, float scale, int32_t topk,
                       int32_t* keep, int64_t keep_stride, int32_t* counts, void* workspace,
                       size_t workspace_bytes, void* stream);
/* 0 for an invalid descriptor or topk < 1. */
size_t kvsel_indexer_topk_workspace_bytes(const kvsel_paged_kv* kv, int32_t num_q_heads, int32_t topk);

/* ------------------------------------------------------------------------
 * Quest page summaries ([LONGCTX] sparse-attention experiment, the Quest
 * strategy: the per-channel minimum and maximum of a page's keys).
 * For every whole page p of every sequence with p >= first_page (pages with
 * (p + 1) * page_size <= L_b; the trailing partial page is never summarised)
 * and every KV head c:
 *   summary[pg][c][0][i] = min over the page's keys k of k[i]
 *   summary[pg][c][1][i] = max over the page's keys k of k[i]
 * where pg = block_table[b][p] is the page's PHYSICAL id, so a summary lives
 * beside its page and stays valid while the page is unchanged: call with
 * first_page = 0 after a prefill and with first_page = the page that just
 * filled after a decode step.  Layout [num_pages][num_kv_heads][2][head_dim]
 * in the cache dtype (min and max of stored values are stored values, so
 * the summary is exact).  Entries of other pages are left untouched.
 * Errors: INVALID (NULL pointers, first_page < 0, bad descriptor),
 * UNSUPPORTED (as the descriptor checks), HIP.
 * ------------------------------------------------------------------------ */
int kvsel_quest_summarize(const kvsel_paged_kv* kv, int32_t first_page, void* summary, void* stream);

/* ------------------------------------------------------------------------
 * Quest selection for one decode query per query head ([LONGCTX]
 * sparse-attention experiment, the Quest strategy).  For sequence b, query
 * head h (KV head c = h / G) and every whole page p < n_b = floor(L_b / P):
 *   bound[b][h][p] = sum_i max(q[b][h][i] * kmin[i], q[b][h][i] * kmax[i])
 * (kmin/kmax: the summary of page block_table[b][p], KV head c; no softmax
 * scale: the order is scale-free).  The min(budget_pages, n_b) pages with the
 * largest bounds are chosen, ties to the lower page, and expanded to their
 * token positions; every token of the partial page [n_b * P, L_b) follows.
 *   summary  as written by kvsel_quest_summarize for every whole page.
 *   q        [num_seqs][num_q_heads][head_dim] (dtype kv->dtype).
 *   bounds   [num_seqs][num_q_heads][bounds_stride] f32 or NULL: receives the
 *            bounds of the whole pages (bounds_stride >= floor(max_seq_len / P)).
 *   out_idx  [num_seqs][num_q_heads][out_stride] i32: ascending positions;
 *            out_stride >= min(budget_pages * P + P - 1, max_seq_len).
 *   out_count[num_seqs][num_q_heads] i32: positions written per row.
 * The index set feeds kvsel_sparse_attn with idx_heads = num_q_heads.
 *   workspace: >= kvsel_quest_workspace_bytes(kv, num_q_heads, budget_pages).
 * Errors: INVALID (NULL pointers, budget_pages < 0, strides too small),
 * UNSUPPORTED (group size not a power of two <= 8 nor a multiple of 8, and
 * the descriptor checks), WORKSPACE, HIP.
 * ------------------------------------------------------------------------ */
int kvsel_quest_select(const kvsel_paged_kv* kv, const void* summary, const void* q,
                       int32_t num_q_heads, int32_t budget_pages, float* bounds,
                       int64_t bounds_stride, int32_t* out_idx, int64_t out_stride,
                       int32_t* out_count, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Quest selection with the causal cut applied after the choice ([LONGCTX]
 * sparse-attention experiment, the Quest strategy as its code states it: the
 * pages are ranked among ALL whole pages of the prompt, the trailing partial
 * page is always taken, and only then are positions after the query
 * dropped).  Identical to kvsel_quest_select over the L_b cached positions,
 * followed by keeping only the listed positions <= query_pos[b]; out_count
 * counts what is kept (the list stays ascending).  This is how a prefill
 * chunk's queries use summaries of the whole prompt; kvsel_quest_select is
 * the decode reading (the query is the last position, nothing to cut).
 *   query_pos [num_seqs] i32 device, 0 <= query_pos[b] < L_b (a
 *             precondition; a value >= L_b - 1 cuts nothing).
 * Other arguments, workspace and errors as kvsel_quest_select, plus INVALID
 * for query_pos == NULL.
 * ------------------------------------------------------------------------ */
int kvsel_quest_select_causal(const kvsel_paged_kv* kv, const void* summary, const void* q,
                              int32_t num_q_heads, int32_t budget_pages, const int32_t* query_pos,
                              float* bounds, int64_t bounds_stride, int32_t* out_idx, int64_t out_stride,
                              int32_t* out_count, void* workspace, size_t workspace_bytes, void* stream);

size_t kvsel_quest_workspace_bytes(const kvsel_paged_kv* kv, int32_t num_q_heads, int32_t budget_pages);

/* ------------------------------------------------------------------------
 * H2O decode step with per-step eviction ([EVICT] §4.2 H2O, with the
 * eviction inside the decode loop: the cache never holds more than the
 * budget plus the new token).  Per (sequence b, KV head c) the caller keeps
 * a list of slots: ascending kept positions slots[b][c][0 .. n) with their
 * cumulative scores slot_cum[b][c][..], n = slot_count[b][c].  The new
 * token's K/V must already sit at position L_b - 1 (seq_lens raised).  The
 * call
 *   1. appends position L_b - 1 with score 0 (n += 1);
 *   2. out[b][h] = softmax attention of query head h over the listed
 *      positions of KV head h / G only; probs[b][h][i] = the probability of
 *      slot i (when probs != NULL);
 *   3. slot_cum[b][c][i] = decay * slot_cum + sum over the group of probs;
 *   4. when n > B (B = budgets[b * num_kv_heads + c] when `budgets` is not
 *      NULL, else `budget`): keeps slots [0, min(sinks, n)), [max(n - window,
 *      0), n) and the top max(0, B - forced) of the others by score (ties to
 *      the lower slot, i.e. the lower position), in slot order, and drops the
 *      rest permanently; slot_count becomes the kept count.
 *   budgets   [num_seqs][num_kv_heads] i32 device array or NULL; every entry
 *             must lie in [0, budget] (`budget` is their host-known bound).
 *   slots     [num_seqs][num_kv_heads][slot_stride] i32, slot_cum f32 alike,
 *   slot_count[num_seqs][num_kv_heads] i32; slot_stride >= budget + 1 and
 *             >= sinks + window + 1 (room for the appended token).
 *   out       [num_seqs][num_q_heads][head_dim] f32.
 *   probs     [num_seqs][num_q_heads][slot_stride] f32 or NULL; entries past
 *             the pre-eviction count are left untouched.
 *   workspace >= kvsel_h2o_workspace_bytes(...).
 * Preconditions: listed positions distinct, ascending and < L_b - 1, and
 * slot_count < slot_stride before the call.
 * Errors: INVALID (NULL pointers, negative sinks / window / budget, slot_stride
 * too small), UNSUPPORTED (group size not a power of two <= 8, slot_stride >
 * 2^24, and the descriptor checks), WORKSPACE, HIP.
 * ------------------------------------------------------------------------ */
int kvsel_h2o_step(const kvsel_paged_kv* kv, const void* q, int32_t num_q_heads, float scale,
                   int32_t* slots, float* slot_cum, int32_t* slot_count, int64_t slot_stride,
                   int32_t sinks, int32_t window, int32_t budget, const int32_t* budgets, float decay,
                   float* out, float* probs, void* workspace, size_t workspace_bytes, void* stream);

size_t kvsel_h2o_workspace_bytes(const kvsel_paged_kv* kv, int32_t num_q_heads, int64_t slot_stride,
                                 int32_t sinks, int32_t window, int32_t budget);

/* The bf16 decode pass normalises probabilities in-kernel: each workgroup
 * posts its chunk's log-sum-exp per head, then reads the posts of the other
 * chunks of its (sequence, KV head) row, polling again while some are
 * missing, for at most `microseconds` of the device's constant wall clock
 * (default 40).  A workgroup that stops waiting leaves its chunk to a fix-up
 * pass, so results are exact either way; the bound only caps the time a
 * workgroup can spend waiting when the chunks of its row are not resident
 * together (other work holding compute units).  With 0 only the chunks that
 * find their whole row posted at the first look finish in-kernel (tests use
 * this to exercise the fix-up).  Returns the previous bound, or
 * KVSEL_ERR_INVALID for a value outside [0, 1000000].  Process-wide. */
int32_t kvsel_set_sync_wait_us(int32_t microseconds);

/* Name of a status code (static string). */
/* kvsel_read_probe: one streaming read of `bytes` bytes of device memory
 * with non-temporal 16-byte loads, sixteen workgroups per compute unit.  It gives the
 * read bandwidth reachable on this GPU, the reference for the HBM-bound
 * calls above (the vendor's peak is a pin rate).  Timing is the caller's.
 * The loads are folded with XOR; `out` (one uint32 of device memory) is
 * written only if the fold equals 0x9E3779B9, so with zeroed data nothing is
 * written.  buf 16-byte aligned, bytes a multiple of 16.
 * Errors: INVALID (NULL pointers, misaligned buf, bytes not a multiple of
 * 16), HIP.
 * ------------------------------------------------------------------------ */
int kvsel_read_probe(const void* buf, size_t bytes, uint32_t* out, void* stream);

const char* kvsel_status_string(int status);

/* The message of the last failed call on this thread ("" if none). */
const char* kvsel_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVSEL_H */
