"""ctypes binding of libkvsel.so.

Argument marshalling only: every function checks that the tensors it is
handed have the dtype, device and layout the C ABI documents, passes their
device pointers and the current HIP stream, and turns a non-zero status into
an exception.  Every step of the computation runs in the library's HIP
kernels; there is no fallback.  The library must have been built
(``python attention_score_guided_amd/build.py``): importing this module
without it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# KVSEL_LIBRARY names another build of the same library (the tests load the
# host-AddressSanitizer build this way); there is no fallback either way.
LIB_PATH = os.environ.get("KVSEL_LIBRARY") or os.path.join(HERE, "libkvsel.so")

KVSEL_OK, KVSEL_ERR_INVALID, KVSEL_ERR_UNSUPPORTED, KVSEL_ERR_WORKSPACE, KVSEL_ERR_HIP = 0, -1, -2, -3, -4
KVSEL_F32, KVSEL_BF16, KVSEL_FP8_E4M3 = 0, 1, 2
EMIT_PROBS, EMIT_LOGITS = 0, 1
REDUCE_NONE, REDUCE_SUM = 0, 1
SELECT_ROWS, SELECT_GLOBAL_PERCENTILE = 0, 1
ACC_SUM, ACC_MAX, ACC_WINDOW_MEAN = 0, 1, 2
BLOCK_TOP_P_MEAN, BLOCK_FRAC_ABOVE, BLOCK_ALL_COLD = 0, 1, 2

# Every symbol include/kvsel.h declares.
EXPORTED = (
    "kvsel_decode_attn_scores", "kvsel_decode_attn_scores_agg", "kvsel_decode_workspace_bytes",
    "kvsel_decode_attn_scores_noalloc",
    "kvsel_accumulate",
    "kvsel_block_aggregate", "kvsel_select_keep", "kvsel_select_workspace_bytes",
    "kvsel_snapkv_vote", "kvsel_snapkv_workspace_bytes", "kvsel_sparse_attn",
    "kvsel_sparse_workspace_bytes", "kvsel_quest_summarize", "kvsel_quest_select", "kvsel_quest_select_causal",
    "kvsel_quest_workspace_bytes", "kvsel_accumulate_ex", "kvsel_block_aggregate_ex", "kvsel_select_threshold", "kvsel_block_update", "kvsel_read_probe",
    "kvsel_union_keep", "kvsel_indexer_scores_fp8", "kvsel_indexer_topk", "kvsel_indexer_topk_workspace_bytes",
    "kvsel_h2o_step", "kvsel_h2o_workspace_bytes", "kvsel_set_sync_wait_us",
    "kvsel_status_string", "kvsel_last_error",
)


class KvselError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


class PagedKVDesc(ctypes.Structure):
    _fields_ = [
        ("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("num_seqs", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python attention_score_guided_amd/build.py`")
    lib = ctypes.CDLL(path)
    P, I32, I64, F, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    D = ctypes.POINTER(PagedKVDesc)
    sig = {
        "kvsel_decode_attn_scores": (ctypes.c_int, [D, P, I32, F, P, P, P, I64, I32, P, I64, F, P, SZ, P]),
        "kvsel_decode_attn_scores_agg": (ctypes.c_int, [D, P, I32, F, P, P, P, I64, P, I64, F, I32, P, P, I64, I64,
                                                         P, SZ, P]),
        "kvsel_decode_workspace_bytes": (SZ, [D, I32, I32]),
        "kvsel_decode_attn_scores_noalloc": (ctypes.c_int, [D, P, I32, F, P, P, P, I64, I32, P, I64, F, P]),
        "kvsel_accumulate": (ctypes.c_int, [P, I64, P, I32, I32, I32, I32, F, P, I64, P]),
        "kvsel_block_aggregate": (ctypes.c_int, [P, I64, P, I32, I32, I32, I32, I32, I32, P, P, I64, P]),
        "kvsel_select_keep": (ctypes.c_int, [P, I64, P, I32, I32, I32, I32, P, I32, I32, I32, P, I64, P, P, SZ, P]),
        "kvsel_select_workspace_bytes": (SZ, [I32, I32, I32]),
        "kvsel_snapkv_vote": (ctypes.c_int, [D, P, I32, I32, I32, F, I32, P, I64, P, SZ, P]),
        "kvsel_snapkv_workspace_bytes": (SZ, [D, I32, I32]),
        "kvsel_sparse_attn": (ctypes.c_int, [D, P, I32, P, I64, P, I32, I32, F, P, P, P, SZ, P]),
        "kvsel_sparse_workspace_bytes": (SZ, [I32, I32, I32, I32]),
        "kvsel_quest_summarize": (ctypes.c_int, [D, I32, P, P]),
        "kvsel_quest_select": (ctypes.c_int, [D, P, P, I32, I32, P, I64, P, I64, P, P, SZ, P]),
        "kvsel_quest_select_causal": (ctypes.c_int, [D, P, P, I32, I32, P, P, I64, P, I64, P, P, SZ, P]),
        "kvsel_quest_workspace_bytes": (SZ, [D, I32, I32]),
        "kvsel_h2o_step": (ctypes.c_int, [D, P, I32, F, P, P, P, I64, I32, I32, I32, P, F, P, P, P, SZ, P]),
        "kvsel_h2o_workspace_bytes": (SZ, [D, I32, I64, I32, I32, I32]),
        "kvsel_accumulate_ex": (ctypes.c_int, [P, I64, P, I32, I32, I32, I32, I32, F, I32, I32, P, P, I64, P]),
        "kvsel_block_aggregate_ex": (ctypes.c_int, [P, I64, P, I32, I32, I32, I32, I32, F, P, I64, P]),
        "kvsel_select_threshold": (ctypes.c_int, [P, I64, P, I32, I32, F, P, I64, P, P]),
        "kvsel_union_keep": (ctypes.c_int, [P, I64, P, I32, I32, I32, I32, P, I64, P, P]),
        "kvsel_indexer_scores_fp8": (ctypes.c_int, [D, P, I32, F, P, I64, P]),
        "kvsel_indexer_topk": (ctypes.c_int, [D, P, I32, F, I32, P, I64, P, P, SZ, P]),
        "kvsel_indexer_topk_workspace_bytes": (SZ, [D, I32, I32]),
        "kvsel_block_update": (ctypes.c_int, [P, I64, P, I32, I32, P, I64, I32, I32, F, P, I64, P]),
        "kvsel_read_probe": (ctypes.c_int, [P, SZ, P, P]),
        "kvsel_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "kvsel_set_sync_wait_us": (I32, [I32]),
        "kvsel_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


_LIB = _load()


def library() -> ctypes.CDLL:
    return _LIB


def _status_name(status: int) -> str:
    return _LIB.kvsel_status_string(status).decode()


def _check(status: int) -> None:
    if status != KVSEL_OK:
        raise KvselError(status, _LIB.kvsel_last_error().decode())


def _ptr(t: Optional[torch.Tensor], dtype=None, name: str = "tensor") -> Optional[int]:
    if t is None:
        return None
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KVSEL_BF16
    if t.dtype == torch.float32:
        return KVSEL_F32
    if t.dtype == torch.float8_e4m3fn:
        return KVSEL_FP8_E4M3
    raise TypeError(f"KV dtype must be bfloat16 or float32, got {t.dtype}")


class PagedKV:
    """Descriptor of one layer's paged cache, holding references to its
    tensors: pages ``[num_pages][H_kv][P][d]``, block table
    ``[B][max_pages]`` int32, lengths ``[B]`` int32."""

    def __init__(self, k_pages: torch.Tensor, v_pages: Optional[torch.Tensor], block_table: torch.Tensor,
                 seq_lens: torch.Tensor, page_size: int, max_seq_len: int):
        self.k_pages, self.v_pages, self.block_table, self.seq_lens = k_pages, v_pages, block_table, seq_lens
        if v_pages is not None and v_pages.dtype != k_pages.dtype:
            raise TypeError("k_pages and v_pages must share a dtype")
        if k_pages.dim() != 4 or k_pages.shape[2] != page_size:
            raise ValueError("k_pages must be [num_pages][H_kv][page_size][head_dim]")
        self.desc = PagedKVDesc(
            _ptr(k_pages, None, "k_pages"), _ptr(v_pages, None, "v_pages"),
            _ptr(block_table, torch.int32, "block_table"), _ptr(seq_lens, torch.int32, "seq_lens"),
            int(block_table.shape[0]), int(k_pages.shape[1]), int(k_pages.shape[3]), int(page_size),
            int(block_table.shape[1]), int(max_seq_len), _dtype_code(k_pages))

    @property
    def dtype(self):
        return self.k_pages.dtype

    def ref(self):
        return ctypes.byref(self.desc)


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]):
    if workspace is None:
        workspace = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


# --------------------------------------------------------------------------
def set_sync_wait_us(microseconds: int) -> int:
    """kvsel_set_sync_wait_us: returns the previous bound (microseconds)."""
    r = int(_LIB.kvsel_set_sync_wait_us(int(microseconds)))
    if r < 0:
        _check(r)
    return r


def decode_workspace_bytes(kv: PagedKV, num_q_heads: int, probs_given: bool) -> int:
    return int(_LIB.kvsel_decode_workspace_bytes(kv.ref(), num_q_heads, int(bool(probs_given))))


NOALLOC_SCRATCH_BYTES = 96 << 20


def decode_attn_scores_noalloc(kv: PagedKV, q: torch.Tensor, num_q_heads: int, scale: float,
                               out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                               probs: Optional[torch.Tensor] = None, emit: int = EMIT_PROBS,
                               cum: Optional[torch.Tensor] = None, decay: float = 1.0, stream=None) -> None:
    """kvsel_decode_attn_scores_noalloc: as decode_attn_scores, with the
    library's static device scratch in place of a workspace (allocates
    nothing, here or in the library)."""
    if q.dtype != kv.dtype:
        raise TypeError("q must have the cache dtype")
    _check(_LIB.kvsel_decode_attn_scores_noalloc(
        kv.ref(), _ptr(q, None, "q"), num_q_heads, float(scale), _ptr(out, torch.float32, "out"),
        _ptr(lse, torch.float32, "lse"), _ptr(probs, torch.float32, "probs"),
        probs.shape[-1] if probs is not None else 0, emit, _ptr(cum, torch.float32, "cum"),
        cum.shape[-1] if cum is not None else 0, float(decay), _stream(stream)))


def decode_attn_scores(kv: PagedKV, q: torch.Tensor, num_q_heads: int, scale: float,
                       out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                       probs: Optional[torch.Tensor] = None, emit: int = EMIT_PROBS,
                       cum: Optional[torch.Tensor] = None, decay: float = 1.0,
                       workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """kvsel_decode_attn_scores (see include/kvsel.h)."""
    if q.dtype != kv.dtype:
        raise TypeError("q must have the cache dtype")
    ws, wsb = _workspace(decode_workspace_bytes(kv, num_q_heads, probs is not None or cum is None),
                         q.device, workspace)
    _check(_LIB.kvsel_decode_attn_scores(
        kv.ref(), _ptr(q, None, "q"), num_q_heads, float(scale),
        _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"),
        _ptr(probs, torch.float32, "probs"), 0 if probs is None else probs.shape[-1], int(emit),
        _ptr(cum, torch.float32, "cum"), 0 if cum is None else cum.shape[-1], float(decay),
        _ptr(ws, None, "workspace"), wsb, _stream(stream)))


def decode_attn_scores_agg(kv: PagedKV, q: torch.Tensor, num_q_heads: int, scale: float,
                           out: Optional[torch.Tensor], lse: Optional[torch.Tensor],
                           probs: Optional[torch.Tensor], cum: torch.Tensor, decay: float,
                           block_size: int, blk_max: Optional[torch.Tensor], blk_mean: Optional[torch.Tensor],
                           blk_head_stride: int, blk_seq_stride: int,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """kvsel_decode_attn_scores_agg: blk_* are flat float32 tensors indexed
    ``b * blk_seq_stride + kvh * blk_head_stride + block`` (or None)."""
    if q.dtype != kv.dtype:
        raise TypeError("q must have the cache dtype")
    ws, wsb = _workspace(decode_workspace_bytes(kv, num_q_heads, probs is not None), q.device, workspace)
    _check(_LIB.kvsel_decode_attn_scores_agg(
        kv.ref(), _ptr(q, None, "q"), num_q_heads, float(scale),
        _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"),
        _ptr(probs, torch.float32, "probs"), 0 if probs is None else probs.shape[-1],
        _ptr(cum, torch.float32, "cum"), cum.shape[-1], float(decay), int(block_size),
        _ptr(blk_max, torch.float32, "blk_max"), _ptr(blk_mean, torch.float32, "blk_mean"),
        int(blk_head_stride), int(blk_seq_stride), _ptr(ws, None, "workspace"), wsb, _stream(stream)))


def accumulate(probs: torch.Tensor, seq_lens: torch.Tensor, num_kv_heads: int, max_seq_len: int,
               cum: torch.Tensor, decay: float = 1.0, stream=None) -> None:
    """kvsel_accumulate: probs ``[B][H_q][stride]``, cum ``[B][H_kv][stride]``."""
    B, Hq, _ = probs.shape
    _check(_LIB.kvsel_accumulate(
        _ptr(probs, torch.float32, "probs"), probs.shape[-1], _ptr(seq_lens, torch.int32, "seq_lens"),
        B, Hq, num_kv_heads, max_seq_len, float(decay), _ptr(cum, torch.float32, "cum"),
        cum.shape[-1], _stream(stream)))


def block_aggregate(scores: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, block_size: int,
                    head_reduce: int = REDUCE_NONE, accumulate: bool = False,
                    out_max: Optional[torch.Tensor] = None, out_mean: Optional[torch.Tensor] = None,
                    stream=None) -> None:
    """kvsel_block_aggregate: scores ``[B][H][stride]``; outputs
    ``[B][H][out_stride]`` (NONE) or ``[B][out_stride]`` (SUM)."""
    B, H, _ = scores.shape
    ref = out_max if out_max is not None else out_mean
    _check(_LIB.kvsel_block_aggregate(
        _ptr(scores, torch.float32, "scores"), scores.shape[-1], _ptr(seq_lens, torch.int32, "seq_lens"),
        B, H, max_seq_len, block_size, int(head_reduce), int(bool(accumulate)),
        _ptr(out_max, torch.float32, "out_max"), _ptr(out_mean, torch.float32, "out_mean"),
        0 if ref is None else ref.shape[-1], _stream(stream)))


def select_workspace_bytes(rows: int, max_len: int, mode: int) -> int:
    return int(_LIB.kvsel_select_workspace_bytes(rows, max_len, mode))


def select_keep(scores: torch.Tensor, lengths: torch.Tensor, max_len: int, sinks: int, window: int,
                budgets: Optional[torch.Tensor], max_budget: int, out_idx: torch.Tensor,
                out_count: torch.Tensor, mode: int = SELECT_ROWS, global_budget: int = 0,
                workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """kvsel_select_keep: scores ``[rows][stride]`` -> out_idx ``[rows][out_stride]``."""
    rows = scores.shape[0]
    ws, wsb = _workspace(select_workspace_bytes(rows, max_len, mode), scores.device, workspace)
    _check(_LIB.kvsel_select_keep(
        _ptr(scores, torch.float32, "scores"), scores.shape[-1], _ptr(lengths, torch.int32, "lengths"),
        rows, max_len, sinks, window, _ptr(budgets, torch.int32, "budgets"), max_budget, int(mode),
        int(global_budget), _ptr(out_idx, torch.int32, "out_idx"), out_idx.shape[-1],
        _ptr(out_count, torch.int32, "out_count"), _ptr(ws, None, "workspace"), wsb, _stream(stream)))


def snapkv_workspace_bytes(kv: PagedKV, num_q_heads: int, window: int) -> int:
    return int(_LIB.kvsel_snapkv_workspace_bytes(kv.ref(), num_q_heads, window))


def snapkv_vote(kv: PagedKV, q_win: torch.Tensor, num_q_heads: int, window: int, pool_kernel: int,
                scale: float, group_reduce: int, votes: torch.Tensor,
                workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """kvsel_snapkv_vote: q_win ``[B][H_q][W][d]`` -> votes ``[B][H][stride]``."""
    ws, wsb = _workspace(snapkv_workspace_bytes(kv, num_q_heads, window), q_win.device, workspace)
    _check(_LIB.kvsel_snapkv_vote(
        kv.ref(), _ptr(q_win, None, "q_win"), num_q_heads, window, pool_kernel, float(scale),
        int(group_reduce), _ptr(votes, torch.float32, "votes"), votes.shape[-1],
        _ptr(ws, None, "workspace"), wsb, _stream(stream)))


def sparse_workspace_bytes(num_seqs: int, num_q_heads: int, head_dim: int, max_count: int) -> int:
    return int(_LIB.kvsel_sparse_workspace_bytes(num_seqs, num_q_heads, head_dim, max_count))


def sparse_attn(kv: PagedKV, q: torch.Tensor, num_q_heads: int, indices: torch.Tensor,
                counts: torch.Tensor, max_count: int, scale: float, out: torch.Tensor,
                probs: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                stream=None) -> None:
    """kvsel_sparse_attn: indices ``[B][idx_heads][stride]``, counts ``[B][idx_heads]``."""
    if q.dtype != kv.dtype:
        raise TypeError("q must have the cache dtype")
    ws, wsb = _workspace(sparse_workspace_bytes(int(q.shape[0]), num_q_heads, int(q.shape[-1]), max_count),
                         q.device, workspace)
    _check(_LIB.kvsel_sparse_attn(
        kv.ref(), _ptr(q, None, "q"), num_q_heads, _ptr(indices, torch.int32, "indices"),
        indices.shape[-1], _ptr(counts, torch.int32, "counts"), int(indices.shape[1]), max_count,
        float(scale), _ptr(out, torch.float32, "out"), _ptr(probs, torch.float32, "probs"),
        _ptr(ws, None, "workspace"), wsb, _stream(stream)))


def quest_summarize(kv: PagedKV, summary: torch.Tensor, first_page: int = 0, stream=None) -> None:
    """kvsel_quest_summarize: summary ``[num_pages][H_kv][2][head_dim]`` in the
    cache dtype (per physical page: channel min, then max)."""
    if summary.dtype != kv.dtype:
        raise TypeError("summary must have the cache dtype")
    _check(_LIB.kvsel_quest_summarize(kv.ref(), int(first_page), _ptr(summary, None, "summary"), _stream(stream)))


def quest_workspace_bytes(kv: PagedKV, num_q_heads: int, budget_pages: int) -> int:
    return int(_LIB.kvsel_quest_workspace_bytes(kv.ref(), num_q_heads, int(budget_pages)))


def quest_select(kv: PagedKV, summary: torch.Tensor, q: torch.Tensor, num_q_heads: int, budget_pages: int,
                 out_idx: torch.Tensor, out_count: torch.Tensor, bounds: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """kvsel_quest_select: out_idx ``[B][H_q][out_stride]``, out_count ``[B][H_q]``,
    bounds ``[B][H_q][bounds_stride]`` or None."""
    if q.dtype != kv.dtype or summary.dtype != kv.dtype:
        raise TypeError("q and summary must have the cache dtype")
    ws, wsb = _workspace(quest_workspace_bytes(kv, num_q_heads, budget_pages), q.device, workspace)
    _check(_LIB.kvsel_quest_select(
        kv.ref(), _ptr(summary, None, "summary"), _ptr(q, None, "q"), num_q_heads, int(budget_pages),
        _ptr(bounds, torch.float32, "bounds"), 0 if bounds is None else bounds.shape[-1],
        _ptr(out_idx, torch.int32, "out_idx"), out_idx.shape[-1], _ptr(out_count, torch.int32, "out_count"),
        _ptr(ws, None, "workspace"), wsb, _stream(stream)))


def quest_select_causal(kv: PagedKV, summary: torch.Tensor, q: torch.Tensor, num_q_heads: int, budget_pages: int,
                        query_pos: torch.Tensor, out_idx: torch.Tensor, out_count: torch.Tensor,
                        bounds: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                        stream=None) -> None:
    """kvsel_quest_select_causal: as quest_select over all cached positions,
    then only positions <= query_pos[b] (``[B]`` int32) are kept."""
    if q.dtype != kv.dtype or summary.dtype != kv.dtype:
        raise TypeError("q and summary must have the cache dtype")
    ws, wsb = _workspace(quest_workspace_bytes(kv, num_q_heads, budget_pages), q.device, workspace)
    _check(_LIB.kvsel_quest_select_causal(
        kv.ref(), _ptr(summary, None, "summary"), _ptr(q, None, "q"), num_q_heads, int(budget_pages),
        _ptr(query_pos, torch.int32, "query_pos"),
        _ptr(bounds, torch.float32, "bounds"), 0 if bounds is None else bounds.shape[-1],
        _ptr(out_idx, torch.int32, "out_idx"), out_idx.shape[-1], _ptr(out_count, torch.int32, "out_count"),
        _ptr(ws, None, "workspace"), wsb, _stream(stream)))


def h2o_workspace_bytes(kv: PagedKV, num_q_heads: int, slot_stride: int, sinks: int, window: int,
                        budget: int) -> int:
    return int(_LIB.kvsel_h2o_workspace_bytes(kv.ref(), num_q_heads, int(slot_stride), int(sinks), int(window),
                                              int(budget)))


def h2o_step(kv: PagedKV, q: torch.Tensor, num_q_heads: int, scale: float, slots: torch.Tensor,
             slot_cum: torch.Tensor, slot_count: torch.Tensor, sinks: int, window: int, budget: int,
             out: torch.Tensor, probs: Optional[torch.Tensor] = None, decay: float = 1.0,
             budgets: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
             stream=None) -> None:
    """kvsel_h2o_step: slots / slot_cum ``[B][H_kv][slot_stride]``, slot_count ``[B][H_kv]``
    (updated in place), out ``[B][H_q][d]``, probs ``[B][H_q][slot_stride]`` or None,
    budgets ``[B][H_kv]`` int32 (each <= budget) or None."""
    if q.dtype != kv.dtype:
        raise TypeError("q must have the cache dtype")
    stride = slots.shape[-1]
    if slot_cum.shape[-1] != stride or (probs is not None and probs.shape[-1] != stride):
        raise ValueError("slots, slot_cum and probs must share the slot stride")
    ws, wsb = _workspace(h2o_workspace_bytes(kv, num_q_heads, stride, sinks, window, budget), q.device, workspace)
    _check(_LIB.kvsel_h2o_step(
        kv.ref(), _ptr(q, None, "q"), num_q_heads, float(scale), _ptr(slots, torch.int32, "slots"),
        _ptr(slot_cum, torch.float32, "slot_cum"), _ptr(slot_count, torch.int32, "slot_count"), stride,
        int(sinks), int(window), int(budget), _ptr(budgets, torch.int32, "budgets"), float(decay),
        _ptr(out, torch.float32, "out"),
        _ptr(probs, torch.float32, "probs"), _ptr(ws, None, "workspace"), wsb, _stream(stream)))


def accumulate_ex(probs: torch.Tensor, seq_lens: torch.Tensor, num_kv_heads: int, max_seq_len: int,
                  cum: torch.Tensor, mode: int, decay: float = 1.0, window: int = 0, step: int = 0,
                  ring: Optional[torch.Tensor] = None, stream=None) -> None:
    """kvsel_accumulate_ex: probs ``[B][H_q][stride]``, cum ``[B][H_kv][stride]``,
    ring ``[window][B][H_kv][stride]`` (WINDOW_MEAN)."""
    B, Hq, _ = probs.shape
    _check(_LIB.kvsel_accumulate_ex(
        _ptr(probs, torch.float32, "probs"), probs.shape[-1], _ptr(seq_lens, torch.int32, "seq_lens"), B, Hq,
        num_kv_heads, max_seq_len, int(mode), float(decay), int(window), int(step),
        _ptr(ring, torch.float32, "ring"), _ptr(cum, torch.float32, "cum"), cum.shape[-1], _stream(stream)))


def block_aggregate_ex(scores: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, block_size: int,
                       mode: int, param: float, out: torch.Tensor, stream=None) -> None:
    """kvsel_block_aggregate_ex: scores ``[B][H][stride]`` -> out ``[B][H][out_stride]``."""
    B, H, _ = scores.shape
    _check(_LIB.kvsel_block_aggregate_ex(
        _ptr(scores, torch.float32, "scores"), scores.shape[-1], _ptr(seq_lens, torch.int32, "seq_lens"), B, H,
        max_seq_len, block_size, int(mode), float(param), _ptr(out, torch.float32, "out"), out.shape[-1],
        _stream(stream)))


def select_threshold(scores: torch.Tensor, lengths: torch.Tensor, max_len: int, threshold: float,
                     out_idx: torch.Tensor, out_count: torch.Tensor, stream=None) -> None:
    """kvsel_select_threshold: scores ``[rows][stride]`` -> out_idx ``[rows][out_stride]``."""
    _check(_LIB.kvsel_select_threshold(
        _ptr(scores, torch.float32, "scores"), scores.shape[-1], _ptr(lengths, torch.int32, "lengths"),
        scores.shape[0], max_len, float(threshold), _ptr(out_idx, torch.int32, "out_idx"), out_idx.shape[-1],
        _ptr(out_count, torch.int32, "out_count"), _stream(stream)))


def union_keep(idx: torch.Tensor, counts: torch.Tensor, num_kv_heads: int, max_len: int, out: torch.Tensor,
               out_count: torch.Tensor, stream=None) -> None:
    """kvsel_union_keep: idx ``[B][H_q][stride]``, counts ``[B][H_q]`` -> out ``[B][H_kv][out_stride]``."""
    B, Hq, _ = idx.shape
    _check(_LIB.kvsel_union_keep(
        _ptr(idx, torch.int32, "idx"), idx.shape[-1], _ptr(counts, torch.int32, "counts"), B, Hq, num_kv_heads,
        max_len, _ptr(out, torch.int32, "out"), out.shape[-1], _ptr(out_count, torch.int32, "out_count"),
        _stream(stream)))


def indexer_scores_fp8(kv: PagedKV, q: torch.Tensor, num_q_heads: int, scale: float, scores: torch.Tensor,
                       stream=None) -> None:
    """kvsel_indexer_scores_fp8: kv pages and q in torch.float8_e4m3fn; scores ``[B][H_q][stride]``."""
    if q.dtype != torch.float8_e4m3fn or kv.dtype != torch.float8_e4m3fn:
        raise TypeError("the FP8 indexer takes float8_e4m3fn pages and queries")
    _check(_LIB.kvsel_indexer_scores_fp8(kv.ref(), _ptr(q, None, "q"), num_q_heads, float(scale),
                                         _ptr(scores, torch.float32, "scores"), scores.shape[-1], _stream(stream)))


def indexer_topk_workspace_bytes(kv: PagedKV, num_q_heads: int, topk: int) -> int:
    return int(_LIB.kvsel_indexer_topk_workspace_bytes(kv.ref(), num_q_heads, topk))


def indexer_topk(kv: PagedKV, q: torch.Tensor, num_q_heads: int, scale: float, topk: int, keep: torch.Tensor,
                 counts: torch.Tensor, workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """kvsel_indexer_topk: indexer pages and q ``[B][H_q][d]``, both bfloat16 or both float8_e4m3fn ->
    keep ``[B*H_q][keep_stride]`` int32 (ascending positions) and counts ``[B*H_q]``."""
    if q.dtype not in (torch.bfloat16, torch.float8_e4m3fn) or q.dtype != kv.dtype:
        raise TypeError("the indexer top-k takes bfloat16 or float8_e4m3fn pages and queries of one dtype")
    ws, wsb = _workspace(indexer_topk_workspace_bytes(kv, num_q_heads, topk), q.device, workspace)
    _check(_LIB.kvsel_indexer_topk(kv.ref(), _ptr(q, None, "q"), num_q_heads, float(scale), int(topk),
                                   _ptr(keep, torch.int32, "keep"), keep.shape[-1],
                                   _ptr(counts, torch.int32, "counts"), _ptr(ws, None, "workspace"), wsb,
                                   _stream(stream)))


def block_meta(rows: int, num_blocks: int, device="cuda") -> torch.Tensor:
    """Zeroed per-block metadata for kvsel_block_update: int32 ``[rows][num_blocks][2]``
    holding kvsel_block_meta records (score bits, stamp); see block_meta_views."""
    return torch.zeros((rows, num_blocks, 2), dtype=torch.int32, device=device)


def block_meta_views(meta: torch.Tensor):
    """(score f32, stamp int32) views ``[rows][num_blocks]`` of a block_meta tensor."""
    return meta.view(torch.float32)[..., 0], meta[..., 1]


def block_update(idx: torch.Tensor, counts: torch.Tensor, block_size: int, step: int, meta: torch.Tensor,
                 values: Optional[torch.Tensor] = None, decay: float = 1.0, stream=None) -> None:
    """kvsel_block_update: idx ``[rows][stride]``, counts ``[rows]``, values aligned with idx
    or None, meta int32 ``[rows][meta_stride][2]`` (block_meta) updated in place."""
    rows, stride = idx.reshape(-1, idx.shape[-1]).shape
    if meta.dim() != 3 or meta.shape[-1] != 2 or meta.shape[0] != rows or not meta.is_contiguous():
        raise ValueError("meta must be a contiguous int32 [rows][meta_stride][2] tensor")
    _check(_LIB.kvsel_block_update(
        _ptr(idx, torch.int32, "idx"), stride, _ptr(counts, torch.int32, "counts"), rows, stride,
        _ptr(values, torch.float32, "values"), 0 if values is None else values.shape[-1], int(block_size),
        int(step), float(decay), _ptr(meta, torch.int32, "meta"), meta.shape[1], _stream(stream)))


def read_probe(buf: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """kvsel_read_probe: one streaming read of the contiguous device tensor ``buf``;
    ``out`` is a one-element int32 device tensor (written only on a sentinel fold)."""
    _check(_LIB.kvsel_read_probe(_ptr(buf, None, "buf"), buf.numel() * buf.element_size(),
                                 _ptr(out, torch.int32, "out"), _stream(stream)))
