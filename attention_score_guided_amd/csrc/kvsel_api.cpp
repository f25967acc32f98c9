// C ABI of libkvsel.so: argument validation (before any HIP call), workspace
// sizing, device check and dispatch to the HIP launchers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/kvsel.h"
#include "kvsel_internal.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return KVSEL_OK;
}

bool is_pow2(long long x) { return x > 0 && (x & (x - 1)) == 0; }

// 0 = unknown, 1 = gfx950, -1 = other.  Indexed by device ordinal.
std::atomic<int> g_arch_ok[64];
// Rate of the device's constant wall clock (kHz), read with the arch check.
std::atomic<int> g_clock_khz[64];

int check_device(int* dev_out = nullptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(KVSEL_ERR_UNSUPPORTED, "no HIP device");
  if (dev < 0 || dev >= 64) return fail(KVSEL_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
  int st = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return fail(KVSEL_ERR_UNSUPPORTED, "cannot query device %d", dev);
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
      khz = 100000;   // the 100 MHz constant clock of CDNA parts
    g_clock_khz[dev].store(khz, std::memory_order_relaxed);
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_arch_ok[dev].store(st, std::memory_order_relaxed);
  }
  if (st != 1) return fail(KVSEL_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  if (dev_out) *dev_out = dev;
  return KVSEL_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(KVSEL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Validation of a paged-KV descriptor shared by every call that reads one.
int check_kv(const kvsel_paged_kv* kv, int32_t num_q_heads, bool need_v) {
  if (!kv) return fail(KVSEL_ERR_INVALID, "kv descriptor is NULL");
  if (!kv->k_pages || !kv->block_table || !kv->seq_lens)
    return fail(KVSEL_ERR_INVALID, "k_pages, block_table and seq_lens are required");
  if (need_v && !kv->v_pages) return fail(KVSEL_ERR_INVALID, "v_pages is required for out");
  if (kv->num_seqs <= 0 || kv->num_kv_heads <= 0 || num_q_heads <= 0 || kv->head_dim <= 0 ||
      kv->page_size <= 0 || kv->max_pages_per_seq <= 0 || kv->max_seq_len <= 0)
    return fail(KVSEL_ERR_INVALID, "dimensions must be positive");
  if (num_q_heads % kv->num_kv_heads != 0)
    return fail(KVSEL_ERR_INVALID, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads,
                kv->num_kv_heads);
  if ((long long)kv->max_pages_per_seq * kv->page_size < kv->max_seq_len)
    return fail(KVSEL_ERR_INVALID, "max_pages_per_seq * page_size < max_seq_len");
  if (kv->head_dim != 64 && kv->head_dim != 128)
    return fail(KVSEL_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", kv->head_dim);
  if (kv->dtype != KVSEL_F32 && kv->dtype != KVSEL_BF16)
    return fail(KVSEL_ERR_UNSUPPORTED, "dtype %d", kv->dtype);
  if (!is_pow2(kv->page_size) || kv->page_size < 16 || kv->page_size > 256)
    return fail(KVSEL_ERR_UNSUPPORTED, "page_size %d (power of two in [16, 256])", kv->page_size);
  return KVSEL_OK;
}

bool group_supported(int g) { return (g <= 8 && is_pow2(g)) || (g > 8 && g % 8 == 0); }

// Per-call tag of the decode pass's row arrival words.  A call counter times
// an odd constant is a bijection on 32 bits, so words left in a workspace by
// any of the previous 2^32 calls never match, and the scattered values make
// a chance match with whatever a fresh workspace holds unlikely (2^-32).
std::atomic<uint32_t> g_calls{0};
uint32_t next_epoch() {
  for (;;) {
    const uint32_t e = (g_calls.fetch_add(1, std::memory_order_relaxed) + 1u) * 0x9E3779B1u;
    if (e != 0) return e;
  }
}

// Bound of the decode pass's wait for the posts of a row, in microseconds of
// the device's constant clock.  A workgroup of the 70B-shape layer runs for
// ~65 us and normally finds its row complete after ~3 us of waiting.
constexpr int kDefaultWaitUs = 40;
std::atomic<int> g_wait_us{kDefaultWaitUs};

// ---- allocation-free decode: the workspace lives in a static device array ----
// Each device that loads the library holds its own copy of `scratch` for the
// life of the process.  In host code the array's name is only a stand-in for
// the symbol: its device address comes from hipGetSymbolAddress, taken once
// per device with that device current and kept here.
static __device__ __align__(256) unsigned char scratch[KVSEL_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];   // per device ordinal, under g_scratch_mu

int scratch_address(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail(KVSEL_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    if (!ptr) return fail(KVSEL_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KVSEL_OK;
}

}  // namespace

extern "C" {

const char* kvsel_status_string(int status) {
  switch (status) {
    case KVSEL_OK: return "KVSEL_OK";
    case KVSEL_ERR_INVALID: return "KVSEL_ERR_INVALID";
    case KVSEL_ERR_UNSUPPORTED: return "KVSEL_ERR_UNSUPPORTED";
    case KVSEL_ERR_WORKSPACE: return "KVSEL_ERR_WORKSPACE";
    case KVSEL_ERR_HIP: return "KVSEL_ERR_HIP";
    default: return "KVSEL_UNKNOWN_STATUS";
  }
}

const char* kvsel_last_error(void) { return g_last_error; }

int32_t kvsel_set_sync_wait_us(int32_t microseconds) {
  if (microseconds < 0) return fail(KVSEL_ERR_INVALID, "wait bound %d us < 0", microseconds);
  if (microseconds > 1000000) return fail(KVSEL_ERR_INVALID, "wait bound %d us > 1 s", microseconds);
  return g_wait_us.exchange(microseconds, std::memory_order_relaxed);
}

size_t kvsel_decode_workspace_bytes(const kvsel_paged_kv* kv, int32_t num_q_heads,
                                    int32_t probs_given) {
  if (check_kv(kv, num_q_heads, false) != KVSEL_OK) return 0;
  return kvsel::plan_decode(kv->num_seqs, kv->num_kv_heads, num_q_heads, kv->head_dim,
                            kv->max_seq_len, probs_given == 0)
      .total_bytes;
}

namespace {

int decode_impl(const kvsel_paged_kv* kv, const void* q, int32_t num_q_heads, float scale, float* out,
                float* lse, float* probs, int64_t probs_stride, int32_t emit, float* cum, int64_t cum_stride,
                float decay, int32_t block_size, float* blk_max, float* blk_mean, int64_t blk_head_stride,
                int64_t blk_seq_stride, void* workspace, size_t workspace_bytes, void* stream,
                bool static_scratch = false) {
  int st = check_kv(kv, num_q_heads, out != nullptr);
  if (st != KVSEL_OK) return st;
  if (!q) return fail(KVSEL_ERR_INVALID, "q is NULL");
  if (emit != KVSEL_EMIT_PROBS && emit != KVSEL_EMIT_LOGITS)
    return fail(KVSEL_ERR_INVALID, "emit %d", emit);
  if (probs && probs_stride < kv->max_seq_len)
    return fail(KVSEL_ERR_INVALID, "probs_stride %lld < max_seq_len %d", (long long)probs_stride,
                kv->max_seq_len);
  if (cum && cum_stride < kv->max_seq_len)
    return fail(KVSEL_ERR_INVALID, "cum_stride %lld < max_seq_len %d", (long long)cum_stride,
                kv->max_seq_len);
  if (emit == KVSEL_EMIT_LOGITS && cum)
    return fail(KVSEL_ERR_UNSUPPORTED, "cum needs probabilities (emit = PROBS)");
  if (!group_supported(num_q_heads / kv->num_kv_heads))
    return fail(KVSEL_ERR_UNSUPPORTED, "group size %d (power of two <= 8 or multiple of 8)",
                num_q_heads / kv->num_kv_heads);
  // The logits scratch is needed only when probabilities are normalised
  // for cum without a caller probs buffer.
  const bool need_scratch = probs == nullptr && cum != nullptr;
  const kvsel::DecodePlan plan = kvsel::plan_decode(kv->num_seqs, kv->num_kv_heads, num_q_heads,
                                                    kv->head_dim, kv->max_seq_len, need_scratch);
  if (static_scratch) {
    if (plan.total_bytes > (size_t)KVSEL_NOALLOC_SCRATCH_BYTES)
      return fail(KVSEL_ERR_WORKSPACE,
                  "this call needs %zu bytes of scratch; the static scratch holds %zu (use "
                  "kvsel_decode_attn_scores with a workspace)",
                  plan.total_bytes, (size_t)KVSEL_NOALLOC_SCRATCH_BYTES);
  } else if (!workspace || workspace_bytes < plan.total_bytes) {
    return fail(KVSEL_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes,
                plan.total_bytes);
  }
  int dev = 0;
  st = check_device(&dev);
  if (st != KVSEL_OK) return st;
  if (static_scratch) {
    // Nothing in the scratch has to start at zero: the normalisation's posts
    // validate themselves and the combine zeroes them after every pass (the
    // array is zero when the library loads).
    st = scratch_address(dev, &workspace);
    if (st != KVSEL_OK) return st;
  }
  kvsel::DecodeArgs a{};
  a.k_pages = kv->k_pages;
  a.v_pages = kv->v_pages;
  a.block_table = kv->block_table;
  a.seq_lens = kv->seq_lens;
  a.q = q;
  a.num_seqs = kv->num_seqs;
  a.num_kv_heads = kv->num_kv_heads;
  a.num_q_heads = num_q_heads;
  a.head_dim = kv->head_dim;
  a.page_size = kv->page_size;
  a.max_pages = kv->max_pages_per_seq;
  a.max_seq_len = kv->max_seq_len;
  a.bf16 = kv->dtype == KVSEL_BF16;
  a.scale = scale;
  a.out = out;
  a.lse = lse;
  a.probs = probs;
  a.probs_stride = probs_stride;
  a.emit_logits = emit == KVSEL_EMIT_LOGITS;
  a.cum = cum;
  a.cum_stride = cum_stride;
  a.decay = decay;
  a.workspace = workspace;
  a.epoch = next_epoch();
  a.wait_ticks = (unsigned long long)g_wait_us.load(std::memory_order_relaxed) *
                 (unsigned long long)g_clock_khz[dev].load(std::memory_order_relaxed) / 1000ull;
  a.blk_bs = block_size;
  a.blk_max = blk_max;
  a.blk_mean = blk_mean;
  a.blk_head_stride = blk_head_stride;
  a.blk_seq_stride = blk_seq_stride;
  return hip_status(kvsel::launch_decode(a, plan, static_cast<hipStream_t>(stream)),
                    "decode_attn_scores launch");
}

}  // namespace

int kvsel_decode_attn_scores_noalloc(const kvsel_paged_kv* kv, const void* q, int32_t num_q_heads,
                                     float scale, float* out, float* lse, float* probs,
                                     int64_t probs_stride, int32_t emit, float* cum, int64_t cum_stride,
                                     float decay, void* stream) {
  // The workspace variant's checks, then the scratch size, all before any
  // HIP call; the static array takes the caller workspace's place.
  return decode_impl(kv, q, num_q_heads, scale, out, lse, probs, probs_stride, emit, cum, cum_stride, decay,
                     0, nullptr, nullptr, 0, 0, nullptr, 0, stream, /*static_scratch=*/true);
}

int kvsel_decode_attn_scores(const kvsel_paged_kv* kv, const void* q, int32_t num_q_heads,
                             float scale, float* out, float* lse, float* probs,
                             int64_t probs_stride, int32_t emit, float* cum, int64_t cum_stride,
                             float decay, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(kv, q, num_q_heads, scale, out, lse, probs, probs_stride, emit, cum, cum_stride, decay,
                     0, nullptr, nullptr, 0, 0, workspace, workspace_bytes, stream);
}

int kvsel_decode_attn_scores_agg(const kvsel_paged_kv* kv, const void* q, int32_t num_q_heads,
                                 float scale, float* out, float* lse, float* probs,
                                 int64_t probs_stride, float* cum, int64_t cum_stride, float decay,
                                 int32_t block_size, float* blk_max, float* blk_mean,
                                 int64_t blk_head_stride, int64_t blk_seq_stride, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (!kv) return fail(KVSEL_ERR_INVALID, "kv is NULL");
  if (!cum) return fail(KVSEL_ERR_INVALID, "block aggregates need cum");
  if (!blk_max && !blk_mean) return fail(KVSEL_ERR_INVALID, "blk_max and blk_mean are both NULL");
  if (block_size <= 0) return fail(KVSEL_ERR_INVALID, "block_size %d <= 0", block_size);
  if (kv->num_kv_heads <= 0 || kv->max_seq_len <= 0)
    return fail(KVSEL_ERR_INVALID, "dimensions must be positive");
  const long long n_blk = ((long long)kv->max_seq_len + block_size - 1) / block_size;
  if (blk_head_stride < n_blk)
    return fail(KVSEL_ERR_INVALID, "blk_head_stride %lld < %lld blocks", (long long)blk_head_stride, n_blk);
  if (blk_seq_stride < (long long)kv->num_kv_heads * blk_head_stride)
    return fail(KVSEL_ERR_INVALID, "blk_seq_stride %lld < num_kv_heads * blk_head_stride",
                (long long)blk_seq_stride);
  return decode_impl(kv, q, num_q_heads, scale, out, lse, probs, probs_stride, KVSEL_EMIT_PROBS, cum,
                     cum_stride, decay, block_size, blk_max, blk_mean, blk_head_stride, blk_seq_stride,
                     workspace, workspace_bytes, stream);
}

int kvsel_accumulate(const float* probs, int64_t probs_stride, const int32_t* seq_lens,
                     int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t max_seq_len, float decay, float* cum, int64_t cum_stride,
                     void* stream) {
  if (!probs || !seq_lens || !cum) return fail(KVSEL_ERR_INVALID, "NULL pointer argument");
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_seq_len <= 0)
    return fail(KVSEL_ERR_INVALID, "dimensions must be positive");
  if (num_q_heads % num_kv_heads != 0)
    return fail(KVSEL_ERR_INVALID, "num_q_heads is not a multiple of num_kv_heads");
  if (probs_stride < max_seq_len || cum_stride < max_seq_len)
    return fail(KVSEL_ERR_INVALID, "stride < max_seq_len");
  int st = check_device();
  if (st != KVSEL_OK) return st;
  return hip_status(kvsel::launch_accumulate(probs, probs_stride, seq_lens, num_seqs, num_q_heads,
                                             num_kv_heads, max_seq_len, decay, cum, cum_stride,
                                             static_cast<hipStream_t>(stream)),
                    "accumulate launch");
}

int kvsel_block_aggregate(const float* scores, int64_t score_stride, const int32_t* seq_lens,
                          int32_t num_seqs, int32_t num_heads, int32_t max_seq_len,
                          int32_t block_size, int32_t head_reduce, int32_t accumulate,
                          float* out_max, float* out_mean, int64_t out_stride, void* stream) {
  if (!scores || !seq_lens) return fail(KVSEL_ERR_INVALID, "NULL pointer argument");
  if (!out_max && !out_mean) return fail(KVSEL_ERR_INVALID, "no output requested");
  if (num_seqs <= 0 || num_heads <= 0 || max_seq_len <= 0 || block_size <= 0)
    return fail(KVSEL_ERR_INVALID, "dimensions must be positive");
  if (head_reduce != KVSEL_REDUCE_NONE && head_reduce != KVSEL_REDUCE_SUM)
    return fail(KVSEL_ERR_INVALID, "head_reduce %d", head_reduce);
  if (accumulate != 0 && accumulate != 1) return fail(KVSEL_ERR_INVALID, "accumulate %d", accumulate);
  if (score_stride < max_seq_len) return fail(KVSEL_ERR_INVALID, "score_stride < max_seq_len");
  const long long n_blk = ((long long)max_seq_len + block_size - 1) / block_size;
  if (out_stride < n_blk)
    return fail(KVSEL_ERR_INVALID, "out_stride %lld < %lld blocks", (long long)out_stride, n_blk);
  int st = check_device();
  if (st != KVSEL_OK) return st;
  return hip_status(
      kvsel::launch_block_aggregate(scores, score_stride, seq_lens, num_seqs, num_heads,
                                    max_seq_len, block_size, head_reduce == KVSEL_REDUCE_SUM,
                                    accumulate != 0, out_max, out_mean, out_stride, 0,
                                    static_cast<hipStream_t>(stream)),
      "block_aggregate launch");
}

size_t kvsel_select_workspace_bytes(int32_t rows, int32_t max_len, int32_t mode) {
  if (rows <= 0 || max_len <= 0 || (mode != KVSEL_SELECT_ROWS && mode != KVSEL_SELECT_GLOBAL_PERCENTILE))
    return 0;
  return kvsel::select_workspace_bytes(rows, max_len, mode);
}

int kvsel_select_keep(const float* scores, int64_t stride, const int32_t* lengths, int32_t rows,
                      int32_t max_len, int32_t sinks, int32_t window, const int32_t* budgets,
                      int32_t max_budget, int32_t mode, int32_t global_budget, int32_t* out_idx,
                      int64_t out_stride, int32_t* out_count, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (!scores || !lengths || !out_idx || !out_count)
    return fail(KVSEL_ERR_INVALID, "NULL pointer argument");
  if (rows <= 0 || max_len <= 0) return fail(KVSEL_ERR_INVALID, "rows and max_len must be positive");
  if (stride < max_len) return fail(KVSEL_ERR_INVALID, "stride < max_len");
  if (sinks < 0 || window < 0 || max_budget < 0 || global_budget < 0)
    return fail(KVSEL_ERR_INVALID, "sinks, window and budgets must be >= 0");
  if (mode == KVSEL_SELECT_ROWS) {
    const long long need = std::min<long long>(max_len, std::max<long long>(max_budget, (long long)sinks + window));
    if (out_stride < need)
      return fail(KVSEL_ERR_INVALID, "out_stride %lld < %lld", (long long)out_stride, need);
    const size_t wneed = kvsel::select_workspace_bytes(rows, max_len, mode);
    if (wneed && (!workspace || workspace_bytes < wneed))
      return fail(KVSEL_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, wneed);
  } else if (mode == KVSEL_SELECT_GLOBAL_PERCENTILE) {
    if (sinks != 0 || window != 0)
      return fail(KVSEL_ERR_INVALID, "GLOBAL_PERCENTILE takes no sinks or window");
    if (out_stride < max_len) return fail(KVSEL_ERR_INVALID, "out_stride < max_len");
    if (max_len > 8192 || (long long)rows * max_len > (1LL << 20))
      return fail(KVSEL_ERR_UNSUPPORTED, "GLOBAL_PERCENTILE needs max_len <= 8192 and rows * max_len <= 2^20");
    const size_t need = kvsel::select_workspace_bytes(rows, max_len, mode);
    if (!workspace || workspace_bytes < need)
      return fail(KVSEL_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  } else {
    return fail(KVSEL_ERR_INVALID, "mode %d", mode);
  }
  int st = check_device();
  if (st != KVSEL_OK) return st;
  return hip_status(kvsel::launch_select(scores, stride, lengths, rows, max_len, sinks, window,
                                         budgets, max_budget, mode, global_budget, out_idx,
                                         out_stride, out_count, workspace,
                                         static_cast<hipStream_t>(stream)),
                    "select_keep launch");
}

size_t kvsel_sparse_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                    int32_t max_count) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_count < 0) return 0;
  return kvsel::sparse_workspace_bytes(num_seqs, num_q_heads, head_dim, max_count);
}

int kvsel_sparse_attn(const kvsel_paged_kv* kv, const void* q, int32_t num_q_heads,
                      const int32_t* indices, int64_t idx_stride, const int32_t* counts,
                      int32_t idx_heads, int32_t max_count, float scale, float* out,
                      float* probs, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_kv(kv, num_q_heads, true);
  if (st != KVSEL_OK) return st;
  if (!q || !indices || !counts || !out) return fail(KVSEL_ERR_INVALID, "NULL pointer argument");
  if (idx_heads != num_q_heads && idx_heads != kv->num_kv_heads)
    return fail(KVSEL_ERR_INVALID, "idx_heads %d must be num_q_heads or num_kv_heads", idx_heads);
  if (max_count < 0 || idx_stride < max_count)
    return fail(KVSEL_ERR_INVALID, "need 0 <= max_count <= idx_stride");
  if (max_count > (1 << 24)) return fail(KVSEL_ERR_UNSUPPORTED, "max_count %d > 2^24", max_count);
  const int G = num_q_heads / kv->num_kv_heads;
  if (idx_heads != num_q_heads && !(G <= 8 && is_pow2(G)))
    return fail(KVSEL_ERR_UNSUPPORTED, "shared index sets need a group size that is a power of two <= 8");
  const size_t need = kvsel::sparse_workspace_bytes(kv->num_seqs, num_q_heads, kv->head_dim, max_count);
  if (!workspace || workspace_bytes < need)
    return fail(KVSEL_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  st = check_device();
  if (st != KVSEL_OK) return st;
  if (max_count == 0) max_count = 1;  // one (empty) slice still writes out = 0
  kvsel::SparseArgs a{};
  a.k_pages = kv->k_pages;
  a.v_pages = kv->v_pages;
  a.block_table = kv->block_table;
  a.seq_lens = kv->seq_lens;
  a.q = q;
  a.indices = indices;
  a.idx_stride = idx_stride;
  a.counts = counts;
  a.num_seqs = kv->num_seqs;
  a.num_kv_heads = kv->num_kv_heads;
  a.num_q_heads = num_q_heads;
  a.head_dim = kv->head_dim;
  a.page_size = kv->page_size;
  a.max_pages = kv->max_pages_per_seq;
  a.idx_heads = idx_heads;
  a.max_count = max_count;
  a.bf16 = kv->dtype == KVSEL_BF16;
  a.scale = scale;
  a.out = out;
  a.probs = probs;
  a.workspace = workspace;
  return hip_status(kvsel::launch_sparse(a, static_cast<hipStream_t>(stream)), "sparse_attn launch");
}

size_t kvsel_snapkv_workspace_bytes(const kvsel_paged_kv* kv, int32_t num_q_heads, int32_t window) {
  if (check_kv(kv, num_q_heads, false) != KVSEL_OK || window <= 0) return 0;
  return kvsel::snapkv_workspace_bytes(kv->num_seqs, kv->num_kv_heads, num_q_heads, window, kv->max_seq_len);
}

int kvsel_snapkv_vote(const kvsel_paged_kv* kv, const void* q_win, int32_t num_q_heads,
                      int32_t window, int32_t pool_kernel, float scale, int32_t group_reduce,
                      float* votes, int64_t votes_stride, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int st = check_kv(kv, num_q_heads, false);
  if (st != KVSEL_OK) return st;
  if (!q_win || !votes) return fail(KVSEL_ERR_INVALID, "NULL pointer argument");
  if (window <= 0 || window >= kv->max_seq_len)
    return fail(KVSEL_ERR_INVALID, "window %d must lie in [1, max_seq_len)", window);
  if (pool_kernel <= 0 || pool_kernel % 2 == 0)
    return fail(KVSEL_ERR_INVALID, "pool_kernel %d must be odd and positive", pool_kernel);
  if (group_reduce != KVSEL_REDUCE_NONE && group_reduce != KVSEL_REDUCE_SUM)
    return fail(KVSEL_ERR_INVALID, "group_reduce %d", group_reduce);
  if (votes_stride < kv->max_seq_len) return fail(KVSEL_ERR_INVALID, "votes_stride < max_seq_len");
  if (kv->dtype != KVSEL_BF16) return fail(KVSEL_ERR_UNSUPPORTED, "the vote runs on bf16 caches");
  if (window > 64) return fail(KVSEL_ERR_UNSUPPORTED, "window %d > 64", window);
  if (pool_kernel > 17) return fail(KVSEL_ERR_UNSUPPORTED, "pool_kernel %d > 17", pool_kernel);
  const size_t need = kvsel::snapkv_workspace_bytes(kv->num_seqs, kv->num_kv_heads, num_q_heads, window, kv->max_seq_len);
  if (!workspace || workspace_bytes < need)
    return fail(KVSEL_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  st = check_device();
  if (st != KVSEL_OK) return st;
  kvsel::SnapkvArgs a{};
  a.k_pages = kv->k_pages;
  a.block_table = kv->block_table;
  a.seq_lens = kv->seq_lens;
  a.q_win = q_win;
  a.num_seqs = kv->num_seqs;
  a.num_kv_heads = kv->num_kv_heads;
  a.num_q_heads = num_q_heads;
  a.head_dim = kv->head_dim;
  a.page_size = kv->page_size;
  a.max_pages = kv->max_pages_per_seq;
  a.max_seq_len = kv->max_seq_len;
  a.window = window;
  a.pool_kernel = pool_kernel;
  a.group_sum = group_reduce == KVSEL_REDUCE_SUM;
  a.scale = scale;
  a.votes = votes;
  a.votes_stride = votes_stride;
  a.workspace = workspace;
  return hip_status(kvsel::launch_snapkv(a, static_cast<hipStream_t>(stream)), "snapkv_vote launch");
}

int kvsel_accumulate_ex(const float* probs, int64_t probs_stride, const int32_t* seq_lens, int32_t num_seqs,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t max_seq_len, int32_t mode, float decay,
                        int32_t window, int32_t step, float* ring, float* cum, int64_t cum_stride, void* stream) {
  if (!probs || !seq_lens || !cum) return fail(KVSEL_ERR_INVALID, "NULL pointer argument");
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_seq_len <= 0)
    return fail(KVSEL_ERR_INVALID, "dimensions must be positive");
  if (num_q_heads % num_kv_heads != 0)
    return fail(KVSEL_ERR_INVALID, "num_q_heads is not a multiple of num_kv_heads");
  if (probs_stride < max_seq_len || cum_stride < max_seq_len) return fail(KVSEL_ERR_INVALID, "stride < max_seq_len");
  if (mode < KVSEL_ACC_SUM || mode > KVSEL_ACC_WINDOW_MEAN) return fail(KVSEL_ERR_INVALID, "mode %d", mode);
  if (mode == KVSEL_ACC_WINDOW_MEAN && (!ring || window <= 0 || step < 0))
    return fail(KVSEL_ERR_INVALID, "WINDOW_MEAN needs a ring, window > 0 and step >= 0");
  int st = check_device();
  if (st != KVSEL_OK) return st;
  return hip_status(kvsel::launch_accumulate_ex(probs, probs_stride, seq_lens, num_seqs, num_q_heads, num_kv_heads,
                                                max_seq_len, mode, decay, window, step, ring, cum, cum_stride,
                                                static_cast<hipStream_t>(stream)),
                    "accumulate_ex launch");
}

int kvsel_block_aggregate_ex(const float* scores, int64_t score_stride, const int32_t* seq_lens, int32_t num_seqs,
                             int32_t num_heads, int32_t max_seq_len, int32_t block_size, int32_t mode, float param,
                             float* out, int64_t out_stride, void* stream) {
  if (!scores || !seq_lens || !out) return fail(KVSEL_ERR_INVALID, "NULL pointer argument");
  if (num_seqs <= 0 || num_heads <= 0 || max_seq_len <= 0 || block_size <= 0)
    return fail(KVSEL_ERR_INVALID, "dimensions must be positive");
  if (mode < KVSEL_BLOCK_TOP_P_MEAN || mode > KVSEL_BLOCK_ALL_COLD) return fail(KVSEL_ERR_INVALID, "mode %d", mode);
  if (score_stride < max_seq_len) return fail(KVSEL_ERR_INVALID, "score_stride < max_seq_len");
  const long long n_blk = ((long long)max_seq_len + block_size - 1) / block_size;
  if (out_stride < n_blk) return fail(KVSEL_ERR_INVALID, "out_stride %lld < %lld blocks", (long long)out_stride, n_blk);
  if (block_size > 256) return fail(KVSEL_ERR_UNSUPPORTED, "block_size %d > 256", block_size);
  int st = check_device();
  if (st != KVSEL_OK) return st;
  return hip_status(kvsel::launch_block_variant(scores, score_stride, seq_lens, num_seqs, num_heads, max_seq_len,
                                                block_size, mode, param, out, out_stride,
                                                static_cast<hipStream_t>(stream)),
                    "block_aggregate_ex launch");
}

int kvsel_read_probe(const void* buf, size_t bytes, uint32_t* out, void* stream) {
  if (!buf || !out) return fail(KVSEL_ERR_INVALID, "NULL pointer argument");
  if ((reinterpret_cast<uintptr_t>(buf) & 15) != 0 || bytes % 16 != 0)
    return fail(KVSEL_ERR_INVALID, "buf must be 16-byte aligned and bytes a multiple of 16");
  int st = check_device();
  if (st != KVSEL_OK) return st;
  if (bytes == 0) return KVSEL_OK;
  return hip_status(kvsel::launch_read_probe(buf, bytes, out, static_cast<hipStream_t>(stream)), "read_probe launch");
}

int kvsel_block_update(const int32_t* idx, int64_t idx_stride, const int32_t* counts, int32_t rows,
                       int32_t max_count, const float* values, int64_t values_stride, int32_t block_size,
                       int32_t step, float decay, kvsel_block_meta* meta, int64_t meta_stride, void* stream) {
  if (!idx || !counts || !meta) return fail(KVSEL_ERR_INVALID, "NULL pointer argument");
  if (rows <= 0 || block_size <= 0 || max_count < 0 || meta_stride <= 0)
    return fail(KVSEL_ERR_INVALID, "rows, block_size and meta_stride must be positive");
  if (idx_stride < max_count || (values && values_stride < max_count))
    return fail(KVSEL_ERR_INVALID, "idx_stride / values_stride < max_count");
  if (rows > 65535) return fail(KVSEL_ERR_UNSUPPORTED, "rows > 65535");
  int st = check_device();
  if (st != KVSEL_OK) return st;
  return hip_status(kvsel::launch_block_update(idx, idx_stride, counts, rows, max_count, values, values_stride,
                                               block_size, step, decay, meta, meta_stride,
                                               static_cast<hipStream_t>(stream)),
                    "block_update launch");
}

int kvsel_select_threshold(const float* scores, int64_t stride, const int32_t* lengths, int32_t rows, int32_t max_len,
                           float threshold, int32_t* out_idx, int64_t out_stride, int32_t* out_count, void* stream) {
  if (!scores || !lengths || !out_idx || !out_count) return fail(KVSEL_ERR_INVALID, "NULL pointer argument");
  if (rows <= 0 || max_len <= 0) return fail(KVSEL_ERR_INVALID, "rows and max_len must be positive");
  if (stride < max_len || out_stride < max_len) return fail(KVSEL_ERR_INVALID, "stride or out_stride < max_len");
  int st = check_device();
  if (st != KVSEL_OK) return st;
  return hip_status(kvsel::launch_select_threshold(scores, stride, lengths, rows, threshold, out_idx, out_stride,
                                                   out_count, static_cast<hipStream_t>(stream)),
                    "select_threshold launch");
}

int kvsel_union_keep(const int32_t* idx, int64_t idx_stride, const int32_t* counts, int32_t num_seqs,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t max_len, int32_t* out, int64_t out_stride,
                     int32_t* out_count, void* stream) {
  if (!idx || !counts || !out || !out_count) return fail(KVSEL_ERR_INVALID, "NULL pointer argument");
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_len <= 0 || idx_stride <= 0)
    return fail(KVSEL_ERR_INVALID, "dimensions must be positive");
  if (num_q_heads % num_kv_heads != 0)
    return fail(KVSEL_ERR_INVALID, "num_q_heads is not a multiple of num_kv_heads");
  const long long need = std::min<long long>(max_len, (long long)(num_q_heads / num_kv_heads) * idx_stride);
  if (out_stride < need) return fail(KVSEL_ERR_INVALID, "out_stride %lld < %lld", (long long)out_stride, need);
  if (max_len > (1 << 20)) return fail(KVSEL_ERR_UNSUPPORTED, "max_len %d > 2^20", max_len);
  int st = check_device();
  if (st != KVSEL_OK) return st;
  return hip_status(kvsel::launch_union_keep(idx, idx_stride, counts, num_seqs, num_q_heads, num_kv_heads, max_len,
                                             out, out_stride, out_count, static_cast<hipStream_t>(stream)),
                    "union_keep launch");
}

int kvsel_indexer_scores_fp8(const kvsel_paged_kv* kv, const void* q, int32_t num_q_heads, float scale,
                             float* scores, int64_t stride, void* stream) {
  if (!kv) return fail(KVSEL_ERR_INVALID, "kv descriptor is NULL");
  if (kv->dtype != KVSEL_FP8_E4M3) return fail(KVSEL_ERR_INVALID, "dtype %d: the FP8 indexer needs FP8_E4M3", kv->dtype);
  kvsel_paged_kv shape = *kv;
  shape.dtype = KVSEL_BF16;   // the shape checks of the other calls
  int st = check_kv(&shape, num_q_heads, false);
  if (st != KVSEL_OK) return st;
  if (!q || !scores) return fail(KVSEL_ERR_INVALID, "NULL pointer argument");
  if (stride < kv->max_seq_len) return fail(KVSEL_ERR_INVALID, "stride < max_seq_len");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(kv->k_pages)) & 15)
    return fail(KVSEL_ERR_INVALID, "q and k_pages must be 16-byte aligned");
  st = check_device();
  if (st != KVSEL_OK) return st;
  return hip_status(kvsel::launch_indexer_fp8(kv->k_pages, kv->block_table, kv->seq_lens, q, kv->num_seqs,
                                              kv->num_kv_heads, num_q_heads, kv->head_dim, kv->page_size,
                                              kv->max_pages_per_seq, kv->max_seq_len, scale, scores, stride,
                                              static_cast<hipStream_t>(stream)),
                    "indexer_scores_fp8 launch");
}

// The indexer top-k's keys are bf16 or FP8 E4M3; the descriptor's other
// fields take the checks of the other calls.
static int check_indexer_kv(const kvsel_paged_kv* kv, int32_t num_q_heads) {
  if (!kv) return fail(KVSEL_ERR_INVALID, "kv descriptor is NULL");
  if (kv->dtype != KVSEL_BF16 && kv->dtype != KVSEL_FP8_E4M3)
    return fail(KVSEL_ERR_UNSUPPORTED, "dtype %d (the indexer top-k takes BF16 or FP8_E4M3)", kv->dtype);
  kvsel_paged_kv shape = *kv;
  shape.dtype = KVSEL_BF16;
  return check_kv(&shape, num_q_heads, false);
}

size_t kvsel_indexer_topk_workspace_bytes(const kvsel_paged_kv* kv, int32_t num_q_heads, int32_t topk) {
  if (check_indexer_kv(kv, num_q_heads) != KVSEL_OK || topk < 1) return 0;
  return kvsel::indexer_topk_workspace_bytes(kv->num_seqs, num_q_heads, kv->max_seq_len, topk);
}

int kvsel_indexer_topk(const kvsel_paged_kv* kv, const void* q, int32_t num_q_heads, float scale, int32_t topk,
                       int32_t* keep, int64_t keep_stride, int32_t* counts, void* workspace,
                       size_t workspace_bytes, void* stream) {
  int st = check_indexer_kv(kv, num_q_heads);
  if (st != KVSEL_OK) return st;
  if (!q || !keep || !counts) return fail(KVSEL_ERR_INVALID, "NULL pointer argument");
  if (topk < 1) return fail(KVSEL_ERR_INVALID, "topk %d < 1", topk);
  if (keep_stride < std::min<int64_t>(topk, kv->max_seq_len))
    return fail(KVSEL_ERR_INVALID, "keep_stride %lld < min(topk, max_seq_len)", (long long)keep_stride);
  if (kv->dtype == KVSEL_FP8_E4M3 && ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(kv->k_pages)) & 15))
    return fail(KVSEL_ERR_INVALID, "q and k_pages must be 16-byte aligned");
  const int g = num_q_heads / kv->num_kv_heads;
  if (!group_supported(g) || g > 32) return fail(KVSEL_ERR_UNSUPPORTED, "group size %d (power of two <= 8, 16, 24 or 32)", g);
  if ((long long)kv->num_seqs * num_q_heads > (1 << 24))
    return fail(KVSEL_ERR_UNSUPPORTED, "num_seqs * num_q_heads > 2^24");
  const size_t need = kvsel::indexer_topk_workspace_bytes(kv->num_seqs, num_q_heads, kv->max_seq_len, topk);
  if (!workspace || workspace_bytes < need)
    return fail(KVSEL_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  st = check_device();
  if (st != KVSEL_OK) return st;
  kvsel::IndexerTopkArgs a{kv->k_pages, kv->block_table, kv->seq_lens, q, kv->num_seqs, kv->num_kv_heads,
                           num_q_heads, kv->head_dim, kv->page_size, kv->max_pages_per_seq, kv->max_seq_len,
                           scale, topk, keep, keep_stride, counts, workspace};
  a.fp8 = kv->dtype == KVSEL_FP8_E4M3;
  return hip_status(kvsel::launch_indexer_topk(a, static_cast<hipStream_t>(stream)), "indexer_topk launch");
}

int kvsel_quest_summarize(const kvsel_paged_kv* kv, int32_t first_page, void* summary, void* stream) {
  int st = check_kv(kv, kv ? kv->num_kv_heads : 1, false);
  if (st != KVSEL_OK) return st;
  if (!summary) return fail(KVSEL_ERR_INVALID, "summary is NULL");
  if (first_page < 0) return fail(KVSEL_ERR_INVALID, "first_page %d < 0", first_page);
  st = check_device();
  if (st != KVSEL_OK) return st;
  kvsel::QuestArgs a{kv->k_pages, kv->block_table, kv->seq_lens, kv->num_seqs, kv->num_kv_heads,
                     kv->num_kv_heads, kv->head_dim, kv->page_size, kv->max_pages_per_seq,
                     kv->max_seq_len, kv->dtype == KVSEL_BF16};
  return hip_status(kvsel::launch_quest_summary(a, summary, first_page, static_cast<hipStream_t>(stream)),
                    "quest_summarize launch");
}

size_t kvsel_quest_workspace_bytes(const kvsel_paged_kv* kv, int32_t num_q_heads, int32_t budget_pages) {
  if (check_kv(kv, num_q_heads, false) != KVSEL_OK || budget_pages < 0) return 0;
  return kvsel::quest_workspace_bytes(kv->num_seqs, num_q_heads, kv->page_size, kv->max_seq_len, budget_pages);
}

namespace {

int quest_select_impl(const kvsel_paged_kv* kv, const void* summary, const void* q, int32_t num_q_heads,
                      int32_t budget_pages, const int32_t* query_pos, float* bounds, int64_t bounds_stride,
                      int32_t* out_idx, int64_t out_stride, int32_t* out_count, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int st = check_kv(kv, num_q_heads, false);
  if (st != KVSEL_OK) return st;
  if (!summary || !q || !out_idx || !out_count) return fail(KVSEL_ERR_INVALID, "NULL pointer argument");
  if (budget_pages < 0) return fail(KVSEL_ERR_INVALID, "budget_pages %d < 0", budget_pages);
  const long long max_whole = kv->max_seq_len / kv->page_size;
  if (bounds && bounds_stride < max_whole)
    return fail(KVSEL_ERR_INVALID, "bounds_stride %lld < %lld whole pages", (long long)bounds_stride, max_whole);
  const long long need = std::min<long long>((long long)budget_pages * kv->page_size + kv->page_size - 1,
                                             kv->max_seq_len);
  if (out_stride < need)
    return fail(KVSEL_ERR_INVALID, "out_stride %lld < %lld", (long long)out_stride, need);
  if (!group_supported(num_q_heads / kv->num_kv_heads))
    return fail(KVSEL_ERR_UNSUPPORTED, "group size %d (power of two <= 8 or multiple of 8)",
                num_q_heads / kv->num_kv_heads);
  const size_t wneed = kvsel::quest_workspace_bytes(kv->num_seqs, num_q_heads, kv->page_size, kv->max_seq_len,
                                                    budget_pages);
  if (!workspace || workspace_bytes < wneed)
    return fail(KVSEL_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, wneed);
  st = check_device();
  if (st != KVSEL_OK) return st;
  kvsel::QuestArgs a{kv->k_pages, kv->block_table, kv->seq_lens, kv->num_seqs, kv->num_kv_heads,
                     num_q_heads, kv->head_dim, kv->page_size, kv->max_pages_per_seq,
                     kv->max_seq_len, kv->dtype == KVSEL_BF16};
  return hip_status(kvsel::launch_quest_select(a, summary, q, budget_pages, query_pos, bounds, bounds_stride,
                                               out_idx, out_stride, out_count, workspace,
                                               static_cast<hipStream_t>(stream)),
                    "quest_select launch");
}

}  // namespace

int kvsel_quest_select(const kvsel_paged_kv* kv, const void* summary, const void* q, int32_t num_q_heads,
                       int32_t budget_pages, float* bounds, int64_t bounds_stride, int32_t* out_idx,
                       int64_t out_stride, int32_t* out_count, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return quest_select_impl(kv, summary, q, num_q_heads, budget_pages, nullptr, bounds, bounds_stride, out_idx,
                           out_stride, out_count, workspace, workspace_bytes, stream);
}

int kvsel_quest_select_causal(const kvsel_paged_kv* kv, const void* summary, const void* q, int32_t num_q_heads,
                              int32_t budget_pages, const int32_t* query_pos, float* bounds,
                              int64_t bounds_stride, int32_t* out_idx, int64_t out_stride, int32_t* out_count,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!query_pos) return fail(KVSEL_ERR_INVALID, "query_pos is NULL");
  return quest_select_impl(kv, summary, q, num_q_heads, budget_pages, query_pos, bounds, bounds_stride, out_idx,
                           out_stride, out_count, workspace, workspace_bytes, stream);
}

size_t kvsel_h2o_workspace_bytes(const kvsel_paged_kv* kv, int32_t num_q_heads, int64_t slot_stride,
                                 int32_t sinks, int32_t window, int32_t budget) {
  if (check_kv(kv, num_q_heads, false) != KVSEL_OK || slot_stride <= 0 || slot_stride > (1 << 24) || sinks < 0 ||
      window < 0 || budget < 0)
    return 0;
  return kvsel::h2o_workspace_bytes(kv->num_seqs, kv->num_kv_heads, num_q_heads, kv->head_dim, slot_stride, sinks,
                                    window, budget);
}

int kvsel_h2o_step(const kvsel_paged_kv* kv, const void* q, int32_t num_q_heads, float scale, int32_t* slots,
                   float* slot_cum, int32_t* slot_count, int64_t slot_stride, int32_t sinks, int32_t window,
                   int32_t budget, const int32_t* budgets, float decay, float* out, float* probs, void* workspace,
                   size_t workspace_bytes, void* stream) {
  int st = check_kv(kv, num_q_heads, true);
  if (st != KVSEL_OK) return st;
  if (!q || !slots || !slot_cum || !slot_count || !out) return fail(KVSEL_ERR_INVALID, "NULL pointer argument");
  if (sinks < 0 || window < 0 || budget < 0) return fail(KVSEL_ERR_INVALID, "sinks, window and budget must be >= 0");
  if (slot_stride > (1 << 24)) return fail(KVSEL_ERR_UNSUPPORTED, "slot_stride %lld > 2^24", (long long)slot_stride);
  if (slot_stride < (long long)budget + 1 || slot_stride < (long long)sinks + window + 1)
    return fail(KVSEL_ERR_INVALID, "slot_stride %lld < max(budget, sinks + window) + 1", (long long)slot_stride);
  const int G = num_q_heads / kv->num_kv_heads;
  if (!(G <= 8 && is_pow2(G)))
    return fail(KVSEL_ERR_UNSUPPORTED, "group size %d (slot lists are shared by a group: power of two <= 8)", G);
  const size_t need = kvsel::h2o_workspace_bytes(kv->num_seqs, kv->num_kv_heads, num_q_heads, kv->head_dim,
                                                 slot_stride, sinks, window, budget);
  if (!workspace || workspace_bytes < need)
    return fail(KVSEL_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  st = check_device();
  if (st != KVSEL_OK) return st;
  kvsel::H2oArgs a{};
  a.sp.k_pages = kv->k_pages;
  a.sp.v_pages = kv->v_pages;
  a.sp.block_table = kv->block_table;
  a.sp.seq_lens = kv->seq_lens;
  a.sp.q = q;
  a.sp.num_seqs = kv->num_seqs;
  a.sp.num_kv_heads = kv->num_kv_heads;
  a.sp.num_q_heads = num_q_heads;
  a.sp.head_dim = kv->head_dim;
  a.sp.page_size = kv->page_size;
  a.sp.max_pages = kv->max_pages_per_seq;
  a.sp.bf16 = kv->dtype == KVSEL_BF16;
  a.sp.scale = scale;
  a.sp.out = out;
  a.sp.probs = probs;
  a.sp.workspace = workspace;
  a.slots = slots;
  a.slot_cum = slot_cum;
  a.slot_count = slot_count;
  a.slot_stride = slot_stride;
  a.sinks = sinks;
  a.window = window;
  a.budget = budget;
  a.budgets = budgets;
  a.decay = decay;
  return hip_status(kvsel::launch_h2o_step(a, static_cast<hipStream_t>(stream)), "h2o_step launch");
}

}  // extern "C"
