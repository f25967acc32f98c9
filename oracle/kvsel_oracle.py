"""Plain float64 definitions of every step of score-guided KV selection.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Nothing here is tuned:
each function is the textbook definition written out with numpy in float64 so
that a reader can check it against the pages by eye.  Inputs arrive as float64
arrays (bf16 and fp32 data widen to float64 exactly).

Sources (cited by title and section; the three pages are web articles):
  [OFFLOAD]   "Sparse attention x KV-cache offloading: eight questions a
              cross-layer design must answer" (forceinjection.github.io)
  [EVICT]     "KV-cache eviction strategies: from attention sinks to H2O and
              SnapKV" (10100.com article)
  [LONGCTX]   "Long context, KV eviction and sparse attention" (AI-infra
              handbook, serving / long-context chapter, anrans.github.io)

Notation follows the pages: H_q query heads share H_kv key/value heads in
groups of G = H_q / H_kv (query head h reads KV head h // G, the
repeat-interleave used in [LONGCTX] "sparse attention" experiment), head dim d,
softmax scale d^-1/2, sequence length L, page (block) size P.

Parity status: every function below is pinned by tests/test_oracle_pins.py
(closed forms, invariants, library routines, brute force, printed values).
The perplexity and relative-error figures that [LONGCTX] prints come from a
trained model whose weights are not available; they are parity unpinned and
no function here claims to reproduce them.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "fp8_e4m3_bits_to_f64",
    "gather_paged",
    "decode_attention",
    "accumulate",
    "block_aggregate",
    "accumulate_max",
    "accumulate_window",
    "block_top_p_mean",
    "block_fraction_above",
    "block_all_cold",
    "block_update",
    "select_threshold",
    "select_keep",
    "streaming_keep",
    "recent_keep",
    "percentile_keys",
    "global_percentile_select",
    "max_pool_1d",
    "snapkv_vote",
    "snapkv_keep",
    "union_keep",
    "indexer_scores",
    "sparse_attention",
    "h2o_evict_step",
    "relative_error",
    "chunk_causal_attention",
    "attention_flops_per_token",
    "attention_linear_crossover",
    "kv_bytes_per_token",
    "quest_page_summary",
    "quest_page_bounds",
    "quest_page_selection",
    "window_index_set",
    "sink_window_index_set",
]


# --------------------------------------------------------------------------
# data widening and the paged layout
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 bit patterns (uint16) to float64, exactly.

    A bfloat16 value is the upper 16 bits of an IEEE float32.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def fp8_e4m3_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen FP8 E4M3 codes (uint8, OCP layout: sign, 4 exponent bits with
    bias 7, 3 mantissa bits; exponent 0 is subnormal, the all-ones
    exponent-and-mantissa code is NaN, there are no infinities) to float64."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = sign * np.ldexp(m / 8.0, -6)
    out = np.where(e == 0, sub, normal)
    return np.where((e == 0xF) & ((b & 0x7) == 0x7), np.nan, out)


def gather_paged(pages: np.ndarray, block_table_row: np.ndarray, length: int) -> np.ndarray:
    """Logical keys (or values) of one sequence from a paged cache.

    ``pages`` is ``[num_pages][H_kv][P][d]``.  Position j of the sequence lives
    in physical page ``block_table_row[j // P]`` at slot ``j % P`` (the block
    table of paged attention, [EVICT] §1 prerequisites / §5).
    Returns ``[H_kv][length][d]``.
    """
    P = pages.shape[2]
    out = np.empty((pages.shape[1], length, pages.shape[3]), dtype=np.float64)
    for j in range(length):
        out[:, j, :] = pages[int(block_table_row[j // P]), :, j % P, :]
    return out


# --------------------------------------------------------------------------
# O1: decode attention that emits every key's probability
# --------------------------------------------------------------------------
def decode_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray | None, scale: float):
    """One decode query per head against every cached key.

    q ``[H_q][d]``, K and V ``[H_kv][L][d]`` (the current token's key is already
    appended, so the query sees all L keys: the causal rule q_pos >= k_pos of
    the [LONGCTX] sparse-attention experiment).  For head h with KV head
    c = h // G:
        s_j   = scale * q_h . k_{c,j}                 (raw logits)
        p_j   = exp(s_j - max s) / sum_i exp(s_i - max s)
        out_h = sum_j p_j v_{c,j}
        lse_h = max s + ln sum_i exp(s_i - max s)
    The per-key probability p is the signal [OFFLOAD] §1.1/§1.3 says engines
    compute every step and then throw away.
    Returns dict(logits [H_q][L], probs [H_q][L], out [H_q][d] or None, lse [H_q]).
    """
    Hq, d = q.shape
    Hkv, L, _ = K.shape
    assert Hq % Hkv == 0 and L >= 1
    G = Hq // Hkv
    logits = np.empty((Hq, L))
    probs = np.empty((Hq, L))
    lse = np.empty(Hq)
    out = None if V is None else np.empty((Hq, V.shape[2]))
    for h in range(Hq):
        c = h // G
        s = scale * (K[c] @ q[h])
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        logits[h] = s
        probs[h] = e / l
        lse[h] = m + np.log(l)
        if V is not None:
            out[h] = probs[h] @ V[c]
    return {"logits": logits, "probs": probs, "out": out, "lse": lse}


# --------------------------------------------------------------------------
# O2: H2O cumulative importance
# --------------------------------------------------------------------------
def accumulate(cum: np.ndarray, probs: np.ndarray, decay: float = 1.0) -> np.ndarray:
    """Fold one step's probabilities into per-KV-head cumulative scores.

    H2O keeps, for every key position, the sum over decode steps of the
    attention it received ([EVICT] §4.2, "accumulated attention score").  Under
    GQA the G query heads of a group read the same key, so the group's
    probabilities are summed into the one score of that key (cum has one row per
    KV head).  ``decay`` < 1 gives the exponential-decay aggregation of
    [OFFLOAD] §2.1; decay = 1 is H2O's plain sum.
    cum ``[H_kv][L]``, probs ``[H_q][L]`` -> new cum ``[H_kv][L]``.
    """
    Hkv, L = cum.shape
    Hq = probs.shape[0]
    G = Hq // Hkv
    new = decay * cum.astype(np.float64)
    for h in range(Hq):
        new[h // G] += probs[h, :L]
    return new


def accumulate_max(cum: np.ndarray, probs: np.ndarray, decay: float = 1.0) -> np.ndarray:
    """Max pooling across decode steps ([OFFLOAD] §2.1): each position keeps
    the peak of its group-summed probability, cum = max(decay*cum, g)."""
    g = accumulate(np.zeros_like(cum, dtype=np.float64), probs)
    return np.maximum(decay * cum.astype(np.float64), g)


def accumulate_window(history, probs: np.ndarray, Hkv: int, window: int) -> np.ndarray:
    """Sliding-window average across decode steps ([OFFLOAD] §2.1): the mean of
    the group-summed probabilities of the last ``window`` steps, steps before
    the first counting as 0.  ``history`` is the list of earlier steps' group
    sums (``[H_kv][L]`` each, newest last); this step's is appended to it."""
    L = probs.shape[1]
    history.append(accumulate(np.zeros((Hkv, L)), probs))
    last = history[-window:]
    total = np.zeros((Hkv, L))
    for g in last:
        total[:, :g.shape[1]] += g
    return total / window


# --------------------------------------------------------------------------
# O3: token -> block aggregation
# --------------------------------------------------------------------------
def block_aggregate(scores: np.ndarray, length: int, block_size: int):
    """Collapse token scores into per-block scores by max and by mean.

    [OFFLOAD] §3.1: offloading moves blocks of 16-256 tokens, so a token-level
    score needs a block-level summary; max keeps any block holding one key
    token, mean averages it away.  Block n covers positions
    [n*bs, min((n+1)*bs, L)); a partial last block aggregates only its valid
    positions.  scores ``[H][>=L]`` -> (max ``[H][n_blk]``, mean ``[H][n_blk]``).
    """
    H = scores.shape[0]
    n_blk = -(-length // block_size)
    mx = np.empty((H, n_blk))
    mean = np.empty((H, n_blk))
    for h in range(H):
        for n in range(n_blk):
            seg = scores[h, n * block_size:min((n + 1) * block_size, length)]
            mx[h, n] = seg.max()
            mean[h, n] = seg.sum() / len(seg)
    return mx, mean


# --------------------------------------------------------------------------
# O4: keep-set selection (sinks + heavy hitters + recent window)
# --------------------------------------------------------------------------
def block_top_p_mean(scores: np.ndarray, length: int, block_size: int, p: float) -> np.ndarray:
    """Per block, the mean of its m = max(1, ceil(p*n)) largest valid scores
    ([OFFLOAD] §3.1 "top-p%", between the block max (p -> 0) and mean (p = 1))."""
    out = []
    for s in range(0, length, block_size):
        vals = sorted(np.asarray(scores[s:min(s + block_size, length)], dtype=np.float64), reverse=True)
        m = max(1, min(len(vals), math.ceil(p * len(vals))))
        out.append(sum(vals[:m]) / m)
    return np.array(out)


def block_fraction_above(scores: np.ndarray, length: int, block_size: int, threshold: float) -> np.ndarray:
    """Per block, the share of its valid positions scoring >= threshold (blocks
    ranked by their share of important tokens, [EVICT] §5.1)."""
    return np.array([np.mean(np.asarray(scores[s:min(s + block_size, length)]) >= threshold)
                     for s in range(0, length, block_size)])


def block_all_cold(scores: np.ndarray, length: int, block_size: int, threshold: float) -> np.ndarray:
    """1 for a block whose every valid position scores < threshold, else 0
    (only all-cold blocks may be evicted, [EVICT] §5.1)."""
    return np.array([float(all(x < threshold for x in scores[s:min(s + block_size, length)]))
                     for s in range(0, length, block_size)])


def block_update(score: np.ndarray, stamp: np.ndarray, index_list, values, block_size: int, step: int,
                 decay: float = 1.0):
    """Per-block metadata of one decode step ([OFFLOAD] §5.1): every block keeps
    a score accumulator and the step of its last update, and each step walks
    the blocks its selection touched.  A touched block first ages its score by
    decay per step since its stamp (the stamp makes the exponential decay of
    [OFFLOAD] §2.1 lazy), then adds the weights of its selected positions
    (``values`` aligned with ``index_list``; None weighs each position 1), and
    takes the current step as its stamp.  Negative list entries are padding.
    Returns new (score, stamp) arrays; untouched blocks keep both."""
    score = np.array(score, dtype=np.float64)
    stamp = np.array(stamp, dtype=np.int64)
    add = {}
    for i, j in enumerate(index_list):
        if j < 0:
            continue
        b = int(j) // block_size
        add[b] = add.get(b, 0.0) + (1.0 if values is None else float(values[i]))
    for b, s in add.items():
        score[b] = score[b] * decay ** (step - stamp[b]) + s
        stamp[b] = step
    return score, stamp


def select_threshold(scores: np.ndarray, n: int, threshold: float) -> np.ndarray:
    """Absolute-threshold selection ([OFFLOAD] §3.2): the positions scoring
    >= threshold, ascending."""
    return np.array([j for j in range(n) if scores[j] >= threshold], dtype=np.int64)


def select_keep(scores: np.ndarray, n: int, sinks: int, window: int, budget: int) -> np.ndarray:
    """H2O keep set of one row: sinks, heavy hitters and the recent window.

    [EVICT] §4.2 pseudocode: the first ``sinks`` positions and the last
    ``window`` positions are never evicted; among the middle positions the
    top-(budget - sinks - window) cumulative scores are the heavy hitters.
    Readings where the page is silent:
      * ``budget >= n`` keeps everything (no eviction needed);
      * the forced sets are always kept, even past the budget, and the number
        of heavy hitters is max(0, budget - |forced|);
      * ``window = 0`` means the middle runs to the end of the row;
      * equal scores: the lower position wins; -0.0 equals +0.0.
    Returns the kept positions, ascending (int64).
    """
    sc = np.asarray(scores[:n], dtype=np.float64)
    assert not np.isnan(sc).any(), "scores must not be NaN"
    if budget >= n:
        return np.arange(n, dtype=np.int64)
    lo = min(sinks, n)
    hi = max(n - window, 0)
    forced = set(range(lo)) | set(range(hi, n))
    k = max(0, budget - len(forced))
    middle = list(range(lo, hi))
    middle.sort(key=lambda j: (-sc[j], j))
    kept = forced | set(middle[:k])
    return np.array(sorted(kept), dtype=np.int64)


def streaming_keep(n: int, budget: int, sinks: int = 4) -> np.ndarray:
    """StreamingLLM keep list: the first ``sinks`` positions plus the most
    recent ``budget - sinks`` ([EVICT] §4.1; [LONGCTX] StreamingLLM experiment,
    "first 4 + recent window" policy).  Applies only once n exceeds the budget."""
    if n <= budget:
        return np.arange(n, dtype=np.int64)
    return np.array(list(range(sinks)) + list(range(n - (budget - sinks), n)), dtype=np.int64)


def recent_keep(n: int, budget: int) -> np.ndarray:
    """Sliding window: keep only the last ``budget`` positions ([EVICT] §2.1;
    [LONGCTX] StreamingLLM experiment, "recent only" policy)."""
    if n <= budget:
        return np.arange(n, dtype=np.int64)
    return np.arange(n - budget, n, dtype=np.int64)


# --------------------------------------------------------------------------
# O5: per-request percentile normalisation and a global top-K
# --------------------------------------------------------------------------
def percentile_keys(scores: np.ndarray, n: int) -> list:
    """Percentile of every item within its own request ([OFFLOAD] §3.2).

    Rank rho in [0, n) ascending by score; among equal scores the lower index
    ranks higher.  The key of an item is the exact rational (rho + 1) / n, so
    every request's best item has key 1.
    Returns a list of ``Fraction`` of length n.
    """
    sc = [float(x) for x in scores[:n]]
    order = sorted(range(n), key=lambda j: (sc[j], -j))
    keys = [None] * n
    for rho, j in enumerate(order):
        keys[j] = Fraction(rho + 1, n)
    return keys


def global_percentile_select(rows_scores, lengths, global_budget: int):
    """Cross-request block selection on per-request percentiles.

    Every item of every row gets its percentile key; the ``global_budget``
    items with the largest keys are kept (ties: lower row, then lower index).
    Returns one ascending index array per row.
    """
    cand = []
    for r, n in enumerate(lengths):
        keys = percentile_keys(rows_scores[r], n)
        for j in range(n):
            cand.append((keys[j], r, j))
    cand.sort(key=lambda t: (-t[0], t[1], t[2]))
    chosen = cand[:max(0, global_budget)]
    out = [[] for _ in lengths]
    for _, r, j in chosen:
        out[r].append(j)
    return [np.array(sorted(x), dtype=np.int64) for x in out]


# --------------------------------------------------------------------------
# O6: SnapKV observation-window vote
# --------------------------------------------------------------------------
def max_pool_1d(x: np.ndarray, kernel: int) -> np.ndarray:
    """1D max pooling, stride 1, same length, padding ignored ([EVICT] §4.3:
    pooling with kernel 7 keeps the neighbours of a high-vote position)."""
    assert kernel % 2 == 1
    r = kernel // 2
    n = len(x)
    out = np.empty(n)
    for j in range(n):
        out[j] = x[max(0, j - r):min(n, j + r + 1)].max()
    return out


def snapkv_vote(q_win: np.ndarray, K: np.ndarray, scale: float, pool_kernel: int,
                group_sum: bool = True) -> np.ndarray:
    """Observation-window vote of SnapKV ([EVICT] §4.3, steps 2-4).

    q_win ``[H_q][W][d]`` holds the queries of the last W prompt positions
    (L - W + i for window row i); K ``[H_kv][L][d]``.  Each window query takes a
    causal softmax over keys 0 .. L - W + i; the vote of prefix key j < L - W is
    the sum of those probabilities over the W window queries (sum pooling per
    head).  With ``group_sum`` the G query heads of a KV head add their votes
    (the KV head is what is kept); then the vote is max-pooled.
    Returns ``[H_kv or H_q][L - W]``.
    """
    Hq, W, d = q_win.shape
    Hkv, L, _ = K.shape
    G = Hq // Hkv
    n_prefix = L - W
    per_head = np.zeros((Hq, n_prefix))
    for h in range(Hq):
        c = h // G
        for i in range(W):
            t = L - W + i
            s = scale * (K[c, :t + 1] @ q_win[h, i])
            e = np.exp(s - s.max())
            p = e / e.sum()
            per_head[h] += p[:n_prefix]
    if group_sum:
        votes = np.zeros((Hkv, n_prefix))
        for h in range(Hq):
            votes[h // G] += per_head[h]
    else:
        votes = per_head
    return np.stack([max_pool_1d(v, pool_kernel) for v in votes])


def snapkv_keep(pooled_vote: np.ndarray, L: int, W: int, k: int) -> np.ndarray:
    """Kept positions of one head: top-k pooled votes plus the window itself
    ([EVICT] §4.3 step 5)."""
    top = select_keep(pooled_vote, L - W, 0, 0, k)
    return np.concatenate([top, np.arange(L - W, L, dtype=np.int64)])


# --------------------------------------------------------------------------
# O7: lightweight indexer score
# --------------------------------------------------------------------------
def union_keep(index_sets) -> np.ndarray:
    """Positions kept for a KV head under GQA: the union of its query heads'
    picks ([EVICT] §4.3, SnapKV's GQA note), ascending, negatives ignored."""
    kept = set()
    for s in index_sets:
        kept |= {int(j) for j in s if j >= 0}
    return np.array(sorted(kept), dtype=np.int64)


def indexer_scores(q_idx: np.ndarray, K_idx: np.ndarray) -> np.ndarray:
    """Dot-product indexer: score_hj = q_h . k_j over a single indexer key
    head ([LONGCTX] sparse attention: a cheap scorer ranks every past token and
    each query attends only its top 2048).  q_idx ``[H][d_I]``, K_idx
    ``[L][d_I]`` -> ``[H][L]``."""
    return q_idx @ K_idx.T


# --------------------------------------------------------------------------
# O8: sparse attention over an index set
# --------------------------------------------------------------------------
def sparse_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, index_sets, scale: float):
    """Softmax attention restricted to a set of key positions.

    [LONGCTX] sparse-attention experiment: logits outside the selection are set
    to -inf before the softmax, i.e. the softmax runs over the set only.
    ``index_sets[h]`` lists the positions query head h may read (-1 entries are
    padding and ignored).  Returns (out ``[H_q][d]``, list of probability
    arrays aligned with each head's index list, -1 entries receiving 0).
    """
    Hq = q.shape[0]
    Hkv = K.shape[0]
    G = Hq // Hkv
    out = np.zeros((Hq, V.shape[2]))
    probs = []
    for h in range(Hq):
        c = h // G
        idx = np.asarray(index_sets[h], dtype=np.int64)
        valid = idx >= 0
        sel = idx[valid]
        p_full = np.zeros(len(idx))
        if len(sel):
            s = scale * (K[c, sel] @ q[h])
            e = np.exp(s - s.max())
            p = e / e.sum()
            out[h] = p @ V[c, sel]
            p_full[valid] = p
        probs.append(p_full)
    return out, probs


def h2o_evict_step(q: np.ndarray, K: np.ndarray, V: np.ndarray, kept, cum, scale: float, sinks: int,
                   window: int, budget: int, decay: float = 1.0):
    """One decode step of H2O with the eviction inside the decode loop
    ([EVICT] §4.2: attention over the cached keys, scores accumulated per key,
    then sinks + heavy hitters + recent window kept and the rest evicted; here
    the cache is the per-KV-head list of kept positions).

    q ``[H_q][d]``; K, V ``[H_kv][L][d]`` logical, position L-1 being the new
    token; ``kept[c]`` the ascending kept positions of KV head c (all < L-1),
    ``cum[c]`` their scores.  The new position joins every list with score 0,
    every query head attends over its KV head's list only, the group's
    probabilities are folded into the list's scores, and the list is cut back
    with ``select_keep`` applied to the list in slot order.
    Returns (out ``[H_q][d]``, probs per query head aligned with its KV head's
    list after the append, new kept lists, new scores).
    """
    Hq, Hkv, L = q.shape[0], K.shape[0], K.shape[1]
    G = Hq // Hkv
    lists = [np.append(np.asarray(kept[c], dtype=np.int64), L - 1) for c in range(Hkv)]
    scores = [np.append(np.asarray(cum[c], dtype=np.float64), 0.0) for c in range(Hkv)]
    out, probs = sparse_attention(q, K, V, [lists[h // G] for h in range(Hq)], scale)
    new_kept, new_cum = [], []
    for c in range(Hkv):
        folded = accumulate(scores[c][None, :], np.stack(probs[c * G:(c + 1) * G]), decay)[0]
        keep = select_keep(folded, len(folded), sinks, window, budget)
        new_kept.append(lists[c][keep])
        new_cum.append(folded[keep])
    return out, probs, new_kept, new_cum


def chunk_causal_attention(q_chunk: np.ndarray, K_cache: np.ndarray, V_cache: np.ndarray,
                           K_chunk: np.ndarray, V_chunk: np.ndarray, scale: float):
    """Attention of one prompt chunk over the kept cache plus the chunk itself.

    [LONGCTX] StreamingLLM experiment: a chunk of queries is run against the
    cache with a causal mask inside the chunk, so chunk query i sees every
    cached key and chunk keys 0..i.  q_chunk ``[H_q][n][d]``, caches
    ``[H_kv][S][d]``, chunk K/V ``[H_kv][n][d]``.
    Returns (out ``[n][H_q][d]``, probs: list over i of ``[H_q][S + i + 1]``).
    """
    n = q_chunk.shape[1]
    outs, probs = [], []
    for i in range(n):
        K = np.concatenate([K_cache, K_chunk[:, :i + 1]], axis=1)
        V = np.concatenate([V_cache, V_chunk[:, :i + 1]], axis=1)
        r = decode_attention(q_chunk[:, i], K, V, scale)
        outs.append(r["out"])
        probs.append(r["probs"])
    return np.stack(outs), probs


def relative_error(out: np.ndarray, full: np.ndarray) -> float:
    """||out - full||_F / ||full||_F ([LONGCTX] sparse-attention experiment)."""
    return float(np.linalg.norm(out - full) / np.linalg.norm(full))


# --------------------------------------------------------------------------
# index sets of the [LONGCTX] sparse-selection comparison
# --------------------------------------------------------------------------
def window_index_set(qpos: int, budget: int) -> np.ndarray:
    """Recent window: keys qpos-budget+1 .. qpos (causal)."""
    return np.arange(max(0, qpos - budget + 1), qpos + 1, dtype=np.int64)


def sink_window_index_set(qpos: int, budget: int, sinks: int = 4) -> np.ndarray:
    """Sinks 0..sinks-1 plus keys qpos-(budget-sinks)+1 .. qpos (causal)."""
    recent = set(range(max(0, qpos - (budget - sinks) + 1), qpos + 1))
    return np.array(sorted(recent | set(range(min(sinks, qpos + 1)))), dtype=np.int64)


def quest_page_summary(K: np.ndarray, page: int = 16):
    """Per-channel min and max of the keys of every whole page of K (``[L][d]``)
    ([LONGCTX] sparse-attention experiment, Quest): returns (kmin, kmax), each
    ``[L // page][d]``.  The trailing partial page has no summary."""
    n_full = K.shape[0] // page
    kmin = np.empty((n_full, K.shape[1]))
    kmax = np.empty((n_full, K.shape[1]))
    for pg in range(n_full):
        blk = K[pg * page:(pg + 1) * page]
        kmin[pg], kmax[pg] = blk.min(axis=0), blk.max(axis=0)
    return kmin, kmax


def quest_page_bounds(q: np.ndarray, kmin: np.ndarray, kmax: np.ndarray) -> np.ndarray:
    """Upper bound of q.k over each page's keys from its channel min / max:
    bound = sum_d max(q_d*kmin_d, q_d*kmax_d) ([LONGCTX], Quest)."""
    return np.array([np.maximum(q * kmin[pg], q * kmax[pg]).sum() for pg in range(kmin.shape[0])])


def quest_page_selection(q: np.ndarray, K: np.ndarray, qpos: int, budget: int, page: int = 16) -> np.ndarray:
    """Quest page-bound selection for one query of one head.

    Over the whole pages of K (``[L][d]``), each channel's min and max bound the
    score of any key of the page: bound = sum_d max(q_d*kmin_d, q_d*kmax_d).
    The budget // page pages with the largest bounds are chosen; keys of the
    trailing partial page are always included; the causal rule then drops
    keys after qpos.
    """
    L = K.shape[0]
    n_full = L // page
    bounds = quest_page_bounds(q, *quest_page_summary(K, page))
    n_pick = min(budget // page, n_full)
    order = sorted(range(n_full), key=lambda pg: (-bounds[pg], pg))
    keys = set()
    for pg in order[:n_pick]:
        keys |= set(range(pg * page, (pg + 1) * page))
    keys |= set(range(n_full * page, L))
    return np.array(sorted(j for j in keys if j <= qpos), dtype=np.int64)


# --------------------------------------------------------------------------
# cost model of the [LONGCTX] chapter
# --------------------------------------------------------------------------
def attention_flops_per_token(S: int, layers: int, heads: int, head_dim: int) -> float:
    """Attention FLOPs of one token against S cached tokens: 4*S*n_h*d_h per
    layer, half for QK^T and half for PV ([LONGCTX] cost of long context)."""
    return 4.0 * S * heads * head_dim * layers


def attention_linear_crossover(params: float, layers: int, heads: int, head_dim: int) -> float:
    """Context length at which attention FLOPs per token equal the 2*params
    FLOPs of the linear layers ([LONGCTX] cost of long context)."""
    return 2.0 * params / (4.0 * layers * heads * head_dim)


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, bytes_per_elt: int = 2) -> int:
    """K and V of every layer for one token ([LONGCTX] cost of long context)."""
    return 2 * layers * kv_heads * head_dim * bytes_per_elt
