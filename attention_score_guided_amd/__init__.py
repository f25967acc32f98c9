"""MI355X-native score-guided KV selection (library ``libkvsel.so``).

The C ABI lives in ``include/kvsel.h``; this package is its Python binding
(``_lib``) plus the in-tree build script (``build``).  Importing it loads the
built library and fails loudly when it is missing.
"""
from ._lib import (  # noqa: F401
    EMIT_LOGITS, EMIT_PROBS, EXPORTED, KVSEL_BF16, KVSEL_ERR_HIP, KVSEL_ERR_INVALID,
    KVSEL_ERR_UNSUPPORTED, KVSEL_ERR_WORKSPACE, KVSEL_F32, KVSEL_OK, REDUCE_NONE, REDUCE_SUM,
    SELECT_GLOBAL_PERCENTILE, SELECT_ROWS, KvselError, PagedKV, PagedKVDesc, accumulate,
    block_aggregate, decode_attn_scores, decode_attn_scores_agg, decode_workspace_bytes, library,
    decode_attn_scores_noalloc, NOALLOC_SCRATCH_BYTES,
    select_keep, select_workspace_bytes, set_sync_wait_us, snapkv_vote, snapkv_workspace_bytes,
    sparse_attn, sparse_workspace_bytes, quest_summarize, quest_select, quest_select_causal, quest_workspace_bytes,
    h2o_step, h2o_workspace_bytes, accumulate_ex, block_aggregate_ex, select_threshold,
    union_keep, indexer_scores_fp8, indexer_topk, indexer_topk_workspace_bytes, KVSEL_FP8_E4M3, block_update,
    block_meta, block_meta_views, read_probe,
    ACC_SUM, ACC_MAX, ACC_WINDOW_MEAN, BLOCK_TOP_P_MEAN, BLOCK_FRAC_ABOVE, BLOCK_ALL_COLD,
)
