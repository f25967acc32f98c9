#!/usr/bin/env python3
"""Benchmark of the score-guided KV selection hot path on one MI355X.

Workload (default ``llama70b_step``): one full decode step of a LLaMA-70B-shape
model on one GPU -- 80 layers, 64 query / 8 KV heads, head dim 128, bf16 paged
KV (page 64), batch 8 at 32768 tokens (~10.7 GB of KV per sequence, 85.9 GB
per step).  Per layer: score-emitting decode attention with per-key
probabilities emitted and folded into the layer's cumulative scores, then the
block-level aggregation (block 64, max; summed over KV heads and layers).  Per
step: per-request percentile normalisation and the global cross-request top-K
(25% of the 4096 blocks).  All inputs are synthetic, drawn from fixed seeds,
and resident in HBM before the timed region.

Prints ONE JSON line (rank 0).  ``value`` is KV bytes read per step divided
by the measured step time.  ``roofline`` describes the dominant call: the
decode attention of one layer, priced at its algorithmic bytes and timed
with HIP events on the launch stream inside the timed region.
``cpu_baseline`` times the float64 oracle on a bounded sample of the same
workload on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, vendor figure
LAYERS, B, HQ, HKV, D, L, PAGE = 80, 8, 64, 8, 128, 32768, 64
BLOCK, BUDGET_FRAC = 64, 0.25
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_attn_llama70b_layer_traffic.json")
DECODE_SOURCES = ["attention_score_guided_amd/csrc/decode_attn.hip",
                  "attention_score_guided_amd/csrc/device_common.hpp"]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kv_bytes_per_layer() -> int:
    return B * HKV * L * D * 2 * 2          # K and V, bf16


def decode_algorithmic_bytes() -> int:
    """Bytes the method must move for one layer's call: K+V once, the emitted
    probabilities written once, the cumulative scores read and written."""
    return kv_bytes_per_layer() + B * HQ * L * 4 + 2 * B * HKV * L * 4


def source_digest() -> str:
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_entry():
    """Measured HBM bytes per decode call from the committed counter summary,
    or None when absent or taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_digest():
        return None
    return t.get("bytes_per_call")


def setup(torch, K, synth):
    """Allocate and fill 80 layers of paged KV, queries, score buffers."""
    bt, _ = synth.shuffled_block_table(B, L, PAGE, synth.generator(4, "cuda"), "cuda")
    layers = []
    for layer in range(LAYERS):
        cfg = synth.llama70b_layer(layer, device="cuda", block_table=bt)
        kvt = cfg["kv"]
        layers.append((K.PagedKV(kvt.k_pages, kvt.v_pages, kvt.block_table, kvt.seq_lens, PAGE, L),
                       cfg["q"]))
    lens = layers[0][0].seq_lens
    n_blk = L // BLOCK
    bufs = dict(
        out=torch.empty((B, HQ, D), device="cuda"),
        lse=torch.empty((B, HQ), device="cuda"),
        probs=torch.empty((B, HQ, L), device="cuda"),
        cum=torch.zeros((LAYERS, B, HKV, L), device="cuda"),
        # per-layer, per-KV-head block max / mean of the updated cum, the
        # layers stacked as extra heads: [B][LAYERS * HKV][n_blk]
        blk_max=torch.zeros((B, LAYERS * HKV, n_blk), device="cuda"),
        blk_mean=torch.zeros((B, LAYERS * HKV, n_blk), device="cuda"),
        agg_max=torch.zeros((B, n_blk), device="cuda"),
        agg_mean=torch.zeros((B, n_blk), device="cuda"),
        blk_lens=torch.full((B,), n_blk, dtype=torch.int32, device="cuda"),
        keep_idx=torch.empty((B, n_blk), dtype=torch.int32, device="cuda"),
        keep_cnt=torch.empty((B,), dtype=torch.int32, device="cuda"),
        lens=lens,
    )
    bufs["ws_dec"] = torch.empty(K.decode_workspace_bytes(layers[0][0], HQ, True), dtype=torch.uint8,
                                 device="cuda")
    bufs["ws_sel"] = torch.empty(max(256, K.select_workspace_bytes(B, n_blk, K.SELECT_GLOBAL_PERCENTILE)),
                                 dtype=torch.uint8, device="cuda")
    return layers, bufs


def step_decode(K, layers, bufs, scale):
    """Part 1 of a step: score-emitting decode attention of every layer
    (probabilities emitted, cumulative scores updated), with the block max /
    mean of each layer's updated cum produced by the same pass."""
    n_blk = L // BLOCK
    bmax, bmean = bufs["blk_max"].view(-1), bufs["blk_mean"].view(-1)
    for li, (kv, q) in enumerate(layers):
        off = li * HKV * n_blk
        K.decode_attn_scores_agg(kv, q, HQ, scale, bufs["out"], bufs["lse"], bufs["probs"], bufs["cum"][li],
                                 1.0, BLOCK, bmax[off:], bmean[off:], n_blk, LAYERS * HKV * n_blk,
                                 workspace=bufs["ws_dec"])


def step_select(K, layers, bufs):
    """Part 2 of a step: the block scores summed over heads and layers (one
    pass over the stacked per-layer blocks: block size 1, head sum), then the
    per-request percentile and the global top-K of blocks."""
    n_blk = L // BLOCK
    K.block_aggregate(bufs["blk_max"], bufs["blk_lens"], n_blk, 1, K.REDUCE_SUM, False, bufs["agg_max"], None)
    K.block_aggregate(bufs["blk_mean"], bufs["blk_lens"], n_blk, 1, K.REDUCE_SUM, False, bufs["agg_mean"], None)
    K.select_keep(bufs["agg_max"], bufs["blk_lens"], n_blk, 0, 0, None, 0, bufs["keep_idx"],
                  bufs["keep_cnt"], mode=K.SELECT_GLOBAL_PERCENTILE,
                  global_budget=int(BUDGET_FRAC * B * n_blk), workspace=bufs["ws_sel"])


def capture(torch, fn):
    """Capture the launches ``fn`` makes into a HIP graph."""
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return graph


def cpu_baseline(torch, layers, scale, budget_s: float = 20.0):
    """Time the float64 oracle on a bounded sample: whole (sequence, KV head)
    rows of the first layers (gather from pages, bf16 widening, attention of
    the 8 query heads, accumulation, block max/mean), as many rows as fit in
    ``budget_s`` seconds.  Returns the oracle's KV GB/s on that sample."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([t.get("num_threads", 1) for t in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    n_pg = L // PAGE
    t_total, rows, bytes_done = 0.0, 0, 0
    order = [(li, b, c) for li in range(len(layers)) for b in range(B) for c in range(HKV)]
    while t_total < budget_s and rows < len(order):
        li, b, c = order[rows]
        kv, q = layers[li]
        pages = kv.block_table[b, :n_pg].long()
        kp = kv.k_pages[pages, c:c + 1].cpu().view(torch.int16).numpy().view(np.uint16)
        vp = kv.v_pages[pages, c:c + 1].cpu().view(torch.int16).numpy().view(np.uint16)
        qh = q[b, c * 8:(c + 1) * 8].cpu().view(torch.int16).numpy().view(np.uint16)
        ident = np.arange(n_pg)
        t0 = time.perf_counter()
        Kf = O.gather_paged(O.bf16_bits_to_f64(kp), ident, L)
        Vf = O.gather_paged(O.bf16_bits_to_f64(vp), ident, L)
        r = O.decode_attention(O.bf16_bits_to_f64(qh), Kf, Vf, scale)
        cum = O.accumulate(np.zeros((1, L)), r["probs"])
        O.block_aggregate(cum, L, BLOCK)
        t_total += time.perf_counter() - t0
        rows += 1
        bytes_done += L * D * 2 * 2
    # the step's selection: per-request percentiles and the global top 25% of
    # the 8 x 512 block scores (one per step), timed on seeded block scores
    n_blk = L // BLOCK
    blk = np.random.default_rng(0).random((B, n_blk))
    t0 = time.perf_counter()
    O.global_percentile_select([blk[b] for b in range(B)], [n_blk] * B, int(BUDGET_FRAC * B * n_blk))
    t_sel = time.perf_counter() - t0
    # scaled to one step: 640 rows of decode work per selection
    rows_per_step = LAYERS * B * HKV
    t_step = t_total / rows * rows_per_step + t_sel
    return {"value": round(rows_per_step * L * D * 2 * 2 / t_step / 1e9, 4), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{rows} (layer, sequence, KV head) rows from the first layers ({rows * 8} query "
                      f"heads x {L} keys; {rows / 64:.2f} of 80 layers): page gather, bf16 widening, "
                      f"attention, accumulation, block max/mean; {t_total:.1f} s; plus one global "
                      f"percentile top-{int(BUDGET_FRAC * B * n_blk)} selection over {B} x {n_blk} block "
                      f"scores ({t_sel * 1e3:.0f} ms), charged once per {rows_per_step} rows (one step)"}


def counters_mode(torch, K, synth) -> int:
    """Run under ``rocprofv3 --pmc``: three decode calls of one 70B-shape layer
    (same launch configuration as the timed step), then a 1 GiB copy whose
    bytes are known exactly (read 1 GiB, write 1 GiB) to calibrate the
    counters."""
    global LAYERS
    LAYERS = 1
    layers, bufs = setup(torch, K, synth)
    scale = 1.0 / math.sqrt(D)
    for _ in range(3):
        step_decode(K, layers, bufs, scale)
    torch.cuda.synchronize()
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    log("counters mode done: decode x3, copy of 1073741824 bytes")
    return 0


def read_probe(torch, K) -> float:
    """GB/s of the library's streaming read probe over 4 GiB on the current
    GPU (non-temporal 16-byte loads, nothing written), best of three averages
    of 5 runs."""
    x = torch.zeros(1 << 30, dtype=torch.int32, device="cuda")
    o = torch.zeros(1, dtype=torch.int32, device="cuda")
    ms = min(timed(torch, lambda: K.read_probe(x, o), 5) for _ in range(3))
    del x, o
    return (1 << 32) / (ms * 1e-3) / 1e9


def timed(torch, fn, reps: int, warmup: int = 1) -> float:
    """Average milliseconds of ``fn`` over ``reps`` runs (HIP events on the
    current stream, after ``warmup`` untimed runs)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def long_context_workload(torch, K, synth, args) -> dict:
    """128K case: B=4, 32/8 heads, d=128, bf16, page 16, L=131072, planted
    sinks and hot regions.  (i) SnapKV vote (window 32, pool 7, group sum)
    and the top-4096 per KV head; (ii) sparse decode steps: the one-head
    d=64 indexer in logits mode, top-2048 per query head, sparse attention;
    (iii) dense decode over the same cache (out only) for comparison."""
    Bq, HQq, HKVq, Lq, W = 4, 32, 8, 131072, 32
    steps = args.steps
    cfg = synth.long_context_128k(seq_len=Lq, sparse_steps=steps, device="cuda")
    kvt, kit = cfg["kv"], cfg["kv_index"]
    cap = Lq + steps
    kv_k = K.PagedKV(kvt.k_pages, None, kvt.block_table, kvt.seq_lens, 16, Lq)
    votes = torch.zeros((Bq, HKVq, Lq), device="cuda")
    ws_v = torch.empty(K.snapkv_workspace_bytes(kv_k, HQq, W), dtype=torch.uint8, device="cuda")
    vrows = votes.view(Bq * HKVq, Lq)
    vlens = torch.full((Bq * HKVq,), Lq - W, dtype=torch.int32, device="cuda")
    vkeep = torch.empty((Bq * HKVq, 4096), dtype=torch.int32, device="cuda")
    vcnt = torch.empty((Bq * HKVq,), dtype=torch.int32, device="cuda")
    ws_vs = torch.empty(max(256, K.select_workspace_bytes(Bq * HKVq, Lq - W, K.SELECT_ROWS)), dtype=torch.uint8,
                        device="cuda")

    def vote():
        K.snapkv_vote(kv_k, cfg["q_win"], HQq, W, 7, cfg["scale"], K.REDUCE_SUM, votes, workspace=ws_v)

    def vote_select():
        vote()
        K.select_keep(vrows, vlens, Lq - W, 0, 0, None, 4096, vkeep, vcnt, workspace=ws_vs)

    if args.counters:
        # counter-collection mode: three votes and nothing else
        for _ in range(3):
            vote()
        torch.cuda.synchronize()
        log("counters mode done: snapkv vote x3 (128K case)")
        return None
    t_vote = timed(torch, vote, 30, warmup=30)
    t_vote_sel = timed(torch, vote_select, 30, warmup=5)
    k_bytes = Bq * HKVq * Lq * 128 * 2
    vote_flops = 2 * (2.0 * Bq * HQq * W * Lq * 128)       # two passes of Q_win K^T

    # sparse decode steps: lengths grow by one per step (the K/V were drawn
    # ahead); each step's length arrays are made before the timed region, so
    # a step launches only the path's own kernels
    step_lens = [torch.full((Bq,), Lq + s + 1, dtype=torch.int32, device="cuda") for s in range(steps)]
    step_rlens = [torch.full((Bq * HQq,), Lq + s + 1, dtype=torch.int32, device="cuda") for s in range(steps)]
    kv_i_s = [K.PagedKV(kit.k_pages, None, kit.block_table, ls, 16, cap) for ls in step_lens]
    kv_f_s = [K.PagedKV(kvt.k_pages, kvt.v_pages, kvt.block_table, ls, 16, cap) for ls in step_lens]
    # score rows padded to a multiple of 64 positions: 16-byte aligned rows
    # whatever the number of steps (the score stores are 16-byte vectors)
    scores = torch.empty((Bq, HQq, -(-cap // 64) * 64), device="cuda")
    srows = scores.view(Bq * HQq, scores.shape[-1])
    keep = torch.empty((Bq * HQq, 2048), dtype=torch.int32, device="cuda")
    kcnt = torch.empty((Bq * HQq,), dtype=torch.int32, device="cuda")
    out = torch.empty((Bq, HQq, 128), device="cuda")
    ws_d = torch.empty(K.decode_workspace_bytes(kv_i_s[0], HQq, True), dtype=torch.uint8, device="cuda")
    ws_s = torch.empty(K.sparse_workspace_bytes(Bq, HQq, 128, 2048), dtype=torch.uint8, device="cuda")
    ws_k = torch.empty(max(256, K.select_workspace_bytes(Bq * HQq, cap, K.SELECT_ROWS)), dtype=torch.uint8,
                       device="cuda")
    ws_x = torch.empty(K.indexer_topk_workspace_bytes(kv_i_s[0], HQq, 2048), dtype=torch.uint8, device="cuda")

    # a step: the indexer's top-2048 per query head (scores computed where the
    # selection needs them, never stored), then sparse attention over them
    def sparse_step(s):
        K.indexer_topk(kv_i_s[s], cfg["qi_dec"][s], HQq, 1.0, 2048, keep, kcnt, workspace=ws_x)
        K.sparse_attn(kv_f_s[s], cfg["q_dec"][s], HQq, keep.view(Bq, HQq, 2048), kcnt.view(Bq, HQq), 2048,
                      cfg["scale"], out, workspace=ws_s)

    # the same step with the scores written out by the indexer pass and then
    # selected by select_keep (the same keep sets)
    def sparse_step_stored(s):
        K.decode_attn_scores(kv_i_s[s], cfg["qi_dec"][s], HQq, 1.0, None, None, scores, K.EMIT_LOGITS,
                             workspace=ws_d)
        K.select_keep(srows, step_rlens[s], cap, 0, 0, None, 2048, keep, kcnt, workspace=ws_k)
        K.sparse_attn(kv_f_s[s], cfg["q_dec"][s], HQq, keep.view(Bq, HQq, 2048), kcnt.view(Bq, HQq), 2048,
                      cfg["scale"], out, workspace=ws_s)

    sparse_step(0)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for s in range(steps):
        sparse_step(s)
    b.record()
    torch.cuda.synchronize()
    t_sparse = a.elapsed_time(b) / steps
    sparse_step_stored(0)
    torch.cuda.synchronize()
    a.record()
    for s in range(steps):
        sparse_step_stored(s)
    b.record()
    torch.cuda.synchronize()
    t_sparse_stored = a.elapsed_time(b) / steps
    # each step alone after a 512 MB read that evicts the Infinity Cache
    # (256 MB) with clean lines, so that no step reads what an earlier one
    # left there (a write would instead leave 256 MB of dirty lines whose
    # write-back then competes with the step); the median of the per-step
    # event intervals
    flush = torch.ones(128 << 20, device="cuda")
    torch.cuda.synchronize()
    per_step = []
    for s in range(steps):
        flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        sparse_step(s)
        e1.record()
        torch.cuda.synchronize()
        per_step.append(e0.elapsed_time(e1))
    del flush
    t_sparse_flushed = sorted(per_step)[len(per_step) // 2]
    # the same steps replayed from one HIP graph: the path allocates nothing
    # and clears no memory with memsets, so a serving loop can capture it;
    # the replay removes the host's launch gaps between the six kernels
    g_sp = capture(torch, lambda: [sparse_step(s) for s in range(steps)])
    t_sparse_graph = timed(torch, g_sp.replay, 3) / steps
    del g_sp
    # algorithmic bytes of a step: the indexer keys once and the gathered K/V
    # rows; the stored-scores step also writes and reads back the scores
    sparse_bytes = (Bq * Lq * 64 * 2) + Bq * HQq * 2048 * 128 * 2 * 2
    sparse_bytes_stored = sparse_bytes + 2 * Bq * HQq * Lq * 4

    # per-block metadata of the offloading layer: the step's probabilities
    # (emitted by the sparse pass) walked into a float score and an int32
    # stamp per block of 16 for every (sequence, query head) row
    sprobs = torch.empty((Bq, HQq, 2048), device="cuda")
    K.sparse_attn(kv_f_s[0], cfg["q_dec"][0], HQq, keep.view(Bq, HQq, 2048), kcnt.view(Bq, HQq), 2048,
                  cfg["scale"], out, sprobs, workspace=ws_s)
    n_blk = -(-cap // 16)
    bmeta = K.block_meta(Bq * HQq, n_blk)
    sp2 = sprobs.view(Bq * HQq, 2048)
    # a launch of a few microseconds: 10 launches replayed from one HIP graph,
    # so the time is the GPU's and not the Python call rate
    g_bup = capture(torch, lambda: [K.block_update(keep, kcnt, 16, 1, bmeta, sp2, 0.9) for _ in range(10)])
    t_bup = timed(torch, g_bup.replay, 5) / 10
    t_bup_eager = timed(torch, lambda: K.block_update(keep, kcnt, 16, 1, bmeta, sp2, 0.9), 10)
    del sprobs, sp2, bmeta, g_bup
    # the offloading layer's sizing: 256 requests x 2000 blocks of metadata,
    # each step's top-512 blocks per request (block ids, block size 1)
    gen = torch.Generator().manual_seed(77)
    oi = torch.stack([torch.sort(torch.randperm(2000, generator=gen)[:512])[0] for _ in range(256)])
    oi = oi.to(torch.int32).cuda()
    oc = torch.full((256,), 512, dtype=torch.int32, device="cuda")
    ov = torch.rand((256, 512), generator=gen).cuda()
    ometa = K.block_meta(256, 2000)
    g_o = capture(torch, lambda: [K.block_update(oi, oc, 1, 1, ometa, ov, 0.9) for _ in range(10)])
    t_bup_o = timed(torch, g_o.replay, 5) / 10
    del oi, oc, ov, ometa, g_o

    # the same indexer with its keys and queries stored as FP8 E4M3
    kv_i8 = K.PagedKV(kit.k_pages.to(torch.float8_e4m3fn), None, kit.block_table, kv_i_s[0].seq_lens, 16, cap)
    qi8 = cfg["qi_dec"][0].to(torch.float8_e4m3fn)
    t_ix8 = timed(torch, lambda: K.indexer_scores_fp8(kv_i8, qi8, HQq, 1.0, scores), 10)
    # its top-2048 per query head without stored scores (the fused call on FP8 pages)
    ws_x8 = torch.empty(K.indexer_topk_workspace_bytes(kv_i8, HQq, 2048), dtype=torch.uint8, device="cuda")
    t_ixk8 = timed(torch, lambda: K.indexer_topk(kv_i8, qi8, HQq, 1.0, 2048, keep, kcnt, workspace=ws_x8), 10)
    t_ixk16 = timed(torch, lambda: K.indexer_topk(kv_i_s[0], cfg["qi_dec"][0], HQq, 1.0, 2048, keep, kcnt,
                                                  workspace=ws_x), 10)
    del ws_x8
    t_ix16 = timed(torch, lambda: K.decode_attn_scores(kv_i_s[0], cfg["qi_dec"][0], HQq, 1.0, None, None, scores,
                                                       K.EMIT_LOGITS, workspace=ws_d), 10)
    ix_scores_bytes = Bq * HQq * (Lq + 1) * 4
    del kv_i8

    # Quest over the same cache: page summaries at prefill, then sparse decode
    # steps whose index sets are the top-128 pages (2048 keys) by page bound;
    # each step refreshes the summary of the last whole page (the page that
    # fills as tokens are appended)
    QP = 128
    summary = torch.empty((kvt.k_pages.shape[0], HKVq, 2, 128), dtype=torch.bfloat16, device="cuda")
    kv_q0 = K.PagedKV(kvt.k_pages, None, kvt.block_table, kvt.seq_lens, 16, cap)
    t_qsum = timed(torch, lambda: K.quest_summarize(kv_q0, summary), 5)
    qidx = torch.empty((Bq, HQq, QP * 16 + 15), dtype=torch.int32, device="cuda")
    qcnt = torch.empty((Bq, HQq), dtype=torch.int32, device="cuda")
    ws_q = torch.empty(K.quest_workspace_bytes(kv_f_s[0], HQq, QP), dtype=torch.uint8, device="cuda")
    ws_qs = torch.empty(K.sparse_workspace_bytes(Bq, HQq, 128, QP * 16 + 15), dtype=torch.uint8, device="cuda")

    def quest_step(s):
        K.quest_summarize(kv_f_s[s], summary, first_page=(Lq + s + 1) // 16 - 1)
        K.quest_select(kv_f_s[s], summary, cfg["q_dec"][s], HQq, QP, qidx, qcnt, workspace=ws_q)
        K.sparse_attn(kv_f_s[s], cfg["q_dec"][s], HQq, qidx, qcnt, qidx.shape[-1], cfg["scale"], out,
                      workspace=ws_qs)

    quest_step(0)
    torch.cuda.synchronize()
    a.record()
    for s in range(steps):
        quest_step(s)
    b.record()
    torch.cuda.synchronize()
    t_quest = a.elapsed_time(b) / steps
    t_qsel = timed(torch, lambda: K.quest_select(kv_f_s[0], summary, cfg["q_dec"][0], HQq, QP, qidx, qcnt,
                                                 workspace=ws_q), 10)
    n_pg = Lq // 16
    qsel_bytes = Bq * HKVq * n_pg * 2 * 128 * 2 + Bq * HQq * n_pg * 4     # summaries in, bounds out
    quest_bytes = qsel_bytes + Bq * HQq * QP * 16 * 128 * 2 * 2           # + gathered K/V

    # dense decode over the same cache (out only; the current token included)
    kv_f = K.PagedKV(kvt.k_pages, kvt.v_pages, kvt.block_table, kvt.seq_lens, 16, cap)
    ws_dd = torch.empty(K.decode_workspace_bytes(kv_f, HQq, True), dtype=torch.uint8, device="cuda")
    q0 = cfg["q_dec"][0]
    t_dense = timed(torch, lambda: K.decode_attn_scores(kv_f, q0, HQq, cfg["scale"], out, None, None,
                                                        K.EMIT_PROBS, None, 1.0, workspace=ws_dd), 10)
    dense_bytes = Bq * HKVq * Lq * 128 * 2 * 2
    return {
        "metric": "KV GB/s (% HBM peak) for score-emitting decode attn + keep-set select",
        "value": round(dense_bytes / (t_dense * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "long_context_128k", "batch": Bq, "seq_len": Lq, "q_heads": HQq,
                   "kv_heads": HKVq, "head_dim": 128, "page_size": 16, "window": W, "pool_kernel": 7,
                   "vote_top_k": 4096, "index_top_k": 2048},
        "dense_decode_us": round(t_dense * 1e3, 1),
        "vote": {"us": round(t_vote * 1e3, 1), "us_with_top4096": round(t_vote_sel * 1e3, 1),
                 "k_gb_per_s": round(k_bytes / (t_vote * 1e-3) / 1e9, 1),
                 "mfma_tflops": round(vote_flops / (t_vote * 1e-3) / 1e12, 1),
                 "mfma_util_vs_2500_tflops": round(vote_flops / (t_vote * 1e-3) / 2.5e15, 4)},
        "sparse_step": {"us": round(t_sparse * 1e3, 1),
                        "gb_per_s": round(sparse_bytes / (t_sparse * 1e-3) / 1e9, 1),
                        "us_graph": round(t_sparse_graph * 1e3, 1),
                        "us_cache_flushed_median": round(t_sparse_flushed * 1e3, 1),
                        "bytes": sparse_bytes,
                        "us_scores_stored": round(t_sparse_stored * 1e3, 1),
                        "bytes_scores_stored": sparse_bytes_stored},
        "block_update": {"us_graph": round(t_bup * 1e3, 2), "us_eager_calls": round(t_bup_eager * 1e3, 1),
                         "rows": Bq * HQq, "entries_per_row": 2048, "block_size": 16,
                         "offload_sizing_us_graph": round(t_bup_o * 1e3, 2),
                         "offload_sizing": "256 requests x 2000 blocks, top-512 blocks each"},
        "indexer": {"bf16_us": round(t_ix16 * 1e3, 1),
                    "bf16_gb_per_s": round((Bq * (Lq + 1) * 64 * 2 + ix_scores_bytes) / (t_ix16 * 1e-3) / 1e9, 1),
                    "fp8_us": round(t_ix8 * 1e3, 1),
                    "fp8_gb_per_s": round((Bq * (Lq + 1) * 64 + ix_scores_bytes) / (t_ix8 * 1e-3) / 1e9, 1),
                    "top2048_no_stored_scores_bf16_us": round(t_ixk16 * 1e3, 1),
                    "top2048_no_stored_scores_fp8_us": round(t_ixk8 * 1e3, 1)},
        "quest": {"summarize_prefill_us": round(t_qsum * 1e3, 1),
                  "summarize_k_gb_per_s": round(k_bytes / (t_qsum * 1e-3) / 1e9, 1),
                  "select_us": round(t_qsel * 1e3, 1),
                  "select_gb_per_s": round(qsel_bytes / (t_qsel * 1e-3) / 1e9, 1),
                  "step_us": round(t_quest * 1e3, 1),
                  "step_gb_per_s": round(quest_bytes / (t_quest * 1e-3) / 1e9, 1),
                  "pages_per_head": QP},
    }


def llama3_workload(torch, K, synth, args) -> dict:
    """Llama-3-8B-shape layer, B=16, ragged L_b ~ U[8K, 32K]: ``steps``
    decode steps, each appending a token, with the H2O accumulation fused
    (probabilities not emitted); then block aggregation (16: max and mean)
    and the keep set of 20% per (sequence, KV head) with sinks 4 and window
    512."""
    steps = args.steps
    cfg = synth.llama3_8b_layer(steps=steps, device="cuda")
    kvt = cfg["kv"]
    Bq, HQq, HKVq = 16, 32, 8
    base = kvt.seq_lens.clone()
    cap = int(base.max()) + steps
    # score rows span the cache capacity in whole pages (16-byte aligned rows)
    stride = -(-cap // 16) * 16
    # each step appends a token: its lengths are made before the timed region
    kv_s = [K.PagedKV(kvt.k_pages, kvt.v_pages, kvt.block_table, (base + s + 1).to(torch.int32), 16, cap)
            for s in range(steps)]
    kv = kv_s[0]
    cum = torch.zeros((Bq, HKVq, stride), device="cuda")
    out = torch.empty((Bq, HQq, 128), device="cuda")
    ws = torch.empty(K.decode_workspace_bytes(kv, HQq, False), dtype=torch.uint8, device="cuda")
    n_blk = -(-cap // 16)
    bmax = torch.zeros((Bq, HKVq, n_blk), device="cuda")
    bmean = torch.zeros((Bq, HKVq, n_blk), device="cuda")
    rows = cum.view(Bq * HKVq, stride)
    final = (base + steps).to(torch.int32)
    rlens = final.repeat_interleave(HKVq).to(torch.int32)
    budgets = (rlens.double() * 0.2).floor().to(torch.int32)
    mb = int(budgets.max())
    keep = torch.empty((Bq * HKVq, mb), dtype=torch.int32, device="cuda")
    kcnt = torch.empty((Bq * HKVq,), dtype=torch.int32, device="cuda")
    # untimed warm-up of every kernel of the step (into scratch score buffers)
    cum_w = torch.zeros_like(cum)
    for _ in range(2):
        K.decode_attn_scores(kv, cfg["q_steps"][0], HQq, cfg["scale"], out, None, None, K.EMIT_PROBS,
                             cum_w, 1.0, workspace=ws)
    K.block_aggregate(cum_w, final, cap, 16, K.REDUCE_NONE, False, bmax, bmean)
    ws_sel = torch.empty(max(256, K.select_workspace_bytes(Bq * HKVq, cap, K.SELECT_ROWS)), dtype=torch.uint8,
                         device="cuda")
    K.select_keep(cum_w.view(Bq * HKVq, stride), rlens, cap, 4, 512, budgets, mb, keep, kcnt, workspace=ws_sel)
    del cum_w
    torch.cuda.synchronize()
    a, b, c = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    a.record()
    for s in range(steps):
        K.decode_attn_scores(kv_s[s], cfg["q_steps"][s], HQq, cfg["scale"], out, None, None, K.EMIT_PROBS,
                             cum, 1.0, workspace=ws)
    b.record()
    K.block_aggregate(cum, final, cap, 16, K.REDUCE_NONE, False, bmax, bmean)
    K.select_keep(rows, rlens, cap, 4, 512, budgets, mb, keep, kcnt, workspace=ws_sel)
    c.record()
    torch.cuda.synchronize()
    t_dec = a.elapsed_time(b) / steps
    t_sel = b.elapsed_time(c)
    # the aggregation variants on the same rows: one step's probabilities
    # (emitted by one more decode call) folded by max pooling and by a
    # 16-step window mean; block top-p% mean, fraction above and all-cold flag
    # of the block-16 scores; absolute-threshold selection of those blocks
    final_kv = K.PagedKV(kvt.k_pages, kvt.v_pages, kvt.block_table, final, 16, cap)
    probs = torch.empty((Bq, HQq, stride), device="cuda")
    K.decode_attn_scores(final_kv, cfg["q_steps"][steps - 1], HQq, cfg["scale"], out, None, probs, K.EMIT_PROBS,
                         None, 1.0, workspace=torch.empty(K.decode_workspace_bytes(final_kv, HQq, True),
                                                          dtype=torch.uint8, device="cuda"))
    cum_v = cum.clone()
    ring = torch.zeros((16, Bq, HKVq, stride), device="cuda")
    t_max = timed(torch, lambda: K.accumulate_ex(probs, final, HKVq, cap, cum_v, K.ACC_MAX, decay=0.99), 10)
    t_win = timed(torch, lambda: K.accumulate_ex(probs, final, HKVq, cap, cum_v, K.ACC_WINDOW_MEAN, window=16,
                                                 step=3, ring=ring), 10)
    blk_out = torch.empty((Bq, HKVq, n_blk), device="cuda")
    t_topp = timed(torch, lambda: K.block_aggregate_ex(cum, final, cap, 16, K.BLOCK_TOP_P_MEAN, 0.25, blk_out), 10)
    t_frac = timed(torch, lambda: K.block_aggregate_ex(cum, final, cap, 16, K.BLOCK_FRAC_ABOVE, 0.01, blk_out), 10)
    blens = ((final + 15) // 16).repeat_interleave(HKVq).to(torch.int32)
    bidx = torch.empty((Bq * HKVq, n_blk), dtype=torch.int32, device="cuda")
    bcnt = torch.empty((Bq * HKVq,), dtype=torch.int32, device="cuda")
    t_thr = timed(torch, lambda: K.select_threshold(blk_out.view(Bq * HKVq, n_blk), blens, n_blk, 0.5, bidx, bcnt),
                  10)
    tok = float(final.sum()) * HKVq
    variants = {
        "acc_max_us": round(t_max * 1e3, 1),
        "acc_max_gb_per_s": round(tok * (4 * HQq // HKVq + 8) / (t_max * 1e-3) / 1e9, 1),
        "acc_window16_us": round(t_win * 1e3, 1),
        "acc_window16_gb_per_s": round(tok * (4 * HQq // HKVq + 4 + 16 * 4 + 4) / (t_win * 1e-3) / 1e9, 1),
        "block16_top25pct_mean_us": round(t_topp * 1e3, 1),
        "block16_frac_above_us": round(t_frac * 1e3, 1),
        "block16_frac_above_gb_per_s": round(tok * 4 / (t_frac * 1e-3) / 1e9, 1),
        "select_threshold_blocks_us": round(t_thr * 1e3, 1),
    }
    del probs, ring, cum_v

    # keys read per step, averaged over the steps (each step appends one token)
    mean_keys = sum(int(L) for L in base.tolist()) + Bq * (steps + 1) / 2.0
    kv_bytes = mean_keys * HKVq * 128 * 2 * 2
    mass = float(cum.double().sum()) / Bq
    return {
        "metric": "KV GB/s (% HBM peak) for score-emitting decode attn + keep-set select",
        "value": round(kv_bytes / (t_dec * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama3_8b_steps", "batch": Bq, "seq_len": "U[8192,32768]",
                   "q_heads": HQq, "kv_heads": HKVq, "head_dim": 128, "page_size": 16,
                   "block_size": 16, "keep": "0.2 L (sinks 4, window 512)"},
        "decode_us_per_step": round(t_dec * 1e3, 1),
        "aggregate_and_select_us": round(t_sel * 1e3, 1),
        "prob_mass_per_seq": round(mass, 3),
        "aggregation_variants": variants,
    }


def tiny_workload(torch, K, synth, args) -> dict:
    """Tiny case: 1 sequence, 4 query heads on 1 KV head, d=64, fp32, page 16,
    512-token prompt, 16 decode steps with the H2O accumulation fused, then
    block 16 max / mean and the keep set (sinks 4, window 64, budget 128)."""
    cfg = synth.tiny_case(device="cuda")
    kvt = cfg["kv"]
    prompt, steps = cfg["prompt"], cfg["steps"]
    cap = prompt + steps
    kv_s = [K.PagedKV(kvt.k_pages, kvt.v_pages, kvt.block_table,
                      torch.tensor([prompt + s + 1], dtype=torch.int32, device="cuda"), 16, cap) for s in range(steps)]
    cum = torch.zeros((1, 1, cap), device="cuda")
    out = torch.empty((1, 4, 64), device="cuda")
    probs = torch.empty((1, 4, cap), device="cuda")
    ws = torch.empty(K.decode_workspace_bytes(kv_s[-1], 4, True), dtype=torch.uint8, device="cuda")
    n_blk = cap // 16
    bmax = torch.empty((1, 1, n_blk), device="cuda")
    bmean = torch.empty((1, 1, n_blk), device="cuda")
    keep = torch.empty((1, 128), dtype=torch.int32, device="cuda")
    kc = torch.empty((1,), dtype=torch.int32, device="cuda")
    final = torch.tensor([cap], dtype=torch.int32, device="cuda")
    bud = torch.tensor([128], dtype=torch.int32, device="cuda")

    def run():
        cum.zero_()
        for s in range(steps):
            K.decode_attn_scores(kv_s[s], cfg["q_steps"][s], 4, cfg["scale"], out, None, probs, K.EMIT_PROBS, cum,
                                 1.0, workspace=ws)
        K.block_aggregate(cum, final, cap, 16, K.REDUCE_NONE, False, bmax, bmean)
        K.select_keep(cum.view(1, cap), final, cap, 4, 64, bud, 128, keep, kc)
    t = timed(torch, run, 20, warmup=3)
    kv_bytes = sum(prompt + s + 1 for s in range(steps)) * 64 * 4 * 2
    return {
        "metric": "KV GB/s (% HBM peak) for score-emitting decode attn + keep-set select",
        "value": round(kv_bytes / (t * 1e-3) / 1e9, 3), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "higher_is_better": True, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "tiny_case", "prompt": prompt, "q_heads": 4, "kv_heads": 1, "head_dim": 64,
                   "page_size": 16, "block_size": 16, "keep": "sinks 4, window 64, budget 128"},
        "note": "kilobyte-sized and launch-bound: the time per step is the figure",
        "us_per_decode_step": round(t * 1e3 / steps, 1),
        "us_all_steps_plus_select": round(t * 1e3, 1),
    }


def qwen_like_workload(torch, K, synth, args) -> dict:
    """Qwen3-0.6B-like layer (16 / 8 heads, d=128, bf16, page 16): 1600
    tokens in 64-token chunks, causal within each chunk (one pseudo-sequence
    per chunk query), under keep-all, recent-256 and sinks-4 + recent (cut back
    to 256 keys after every chunk); then the last 64 queries under the four
    strategies of the long-context experiment (recent window, sinks + window,
    Quest 16 pages, exact top-256), each against full attention."""
    import numpy as np
    cfg = synth.qwen_like_layer()
    Hkv, N, d = cfg["K"].shape
    Hq, C, budget, scale, P = cfg["num_q_heads"], cfg["chunk"], cfg["budget"], cfg["scale"], 16
    g = synth.generator(21)
    bt, n_pages = synth.shuffled_block_table(1, N, P, g)
    kp = torch.zeros((n_pages, Hkv, P, d), dtype=torch.bfloat16)
    vp = torch.zeros((n_pages, Hkv, P, d), dtype=torch.bfloat16)
    synth.write_positions(kp, bt[0], 0, cfg["K"])
    synth.write_positions(vp, bt[0], 0, cfg["V"])
    kp, vp = kp.cuda(), vp.cuda()
    bt64 = bt.repeat(C, 1).cuda()
    Q = cfg["Q"].cuda()
    chunks = list(range(0, N, C))
    qs = [Q[:, c0:c0 + C].permute(1, 0, 2).contiguous() for c0 in chunks]
    out = torch.empty((C, Hq, d), device="cuda")
    ws_d = torch.empty(K.decode_workspace_bytes(K.PagedKV(kp, vp, bt64, torch.ones(C, dtype=torch.int32,
                                                                                   device="cuda"), P, N), Hq, True),
                       dtype=torch.uint8, device="cuda")
    # keep-all: each chunk's queries against every earlier key
    kv_all = [K.PagedKV(kp, vp, bt64, torch.arange(c0 + 1, c0 + C + 1, dtype=torch.int32, device="cuda"), P,
                        c0 + C) for c0 in chunks]

    def run_all():
        for i in range(len(chunks)):
            K.decode_attn_scores(kv_all[i], qs[i], Hq, scale, out, None, None, K.EMIT_PROBS, workspace=ws_d)
    t_all = timed(torch, run_all, 5) / len(chunks)
    # K+V of the cache each chunk reads (every pseudo-sequence reads the same
    # prefix again, from the caches: the HBM bytes are the cache once)
    kv_bytes = sum(c0 + C for c0 in chunks) * Hkv * d * 2 * 2 / len(chunks)

    # recent-256 / sinks-4 + recent: the index lists of every chunk follow
    # from the policy (the kept keys are the policy's forced sets), so they
    # are made before the timed region; each chunk runs the sparse attention
    # and the cut of its cache back to 256 keys
    stride = budget + C
    ws_s = torch.empty(K.sparse_workspace_bytes(C, Hq, d, stride), dtype=torch.uint8, device="cuda")
    keep = torch.empty((1, budget), dtype=torch.int32, device="cuda")
    kc = torch.empty((1,), dtype=torch.int32, device="cuda")
    zeros = torch.zeros((1, N), device="cuda")
    policy_us = {}
    for name, sinks in [("recent_256", 0), ("sinks_4_recent", 4)]:
        idxs, cnts, lens_c, cut_lens = [], [], [], []
        for c0 in chunks:
            kept = np.arange(c0) if c0 <= budget else np.concatenate(
                [np.arange(min(sinks, c0)), np.arange(c0 - (budget - sinks), c0)])
            idx = np.full((C, Hkv, stride), -1, dtype=np.int32)
            cnt = np.zeros((C, Hkv), dtype=np.int32)
            for i in range(C):
                lst = np.concatenate([kept, np.arange(c0, c0 + i + 1)])
                idx[i, :, :len(lst)] = lst
                cnt[i] = len(lst)
            idxs.append(torch.from_numpy(idx).cuda())
            cnts.append(torch.from_numpy(cnt).cuda())
            lens_c.append(K.PagedKV(kp, vp, bt64, torch.full((C,), c0 + C, dtype=torch.int32, device="cuda"), P,
                                    c0 + C))
            cut_lens.append(torch.tensor([c0 + C], dtype=torch.int32, device="cuda"))

        def run_policy():
            for i, c0 in enumerate(chunks):
                K.sparse_attn(lens_c[i], qs[i], Hq, idxs[i], cnts[i], stride, scale, out, workspace=ws_s)
                K.select_keep(zeros, cut_lens[i], c0 + C, sinks, budget - sinks, None, budget, keep, kc)
        policy_us[name] = round(timed(torch, run_policy, 5) / len(chunks) * 1e3, 1)

    # the last 64 queries: full attention and the four strategies
    pos = np.arange(N - C, N)
    kvl = K.PagedKV(kp, vp, bt64, torch.tensor(pos + 1, dtype=torch.int32, device="cuda"), P, N)
    ql = qs[-1]
    full = torch.empty((C, Hq, d), device="cuda")
    K.decode_attn_scores(kvl, ql, Hq, scale, full, None, None, K.EMIT_PROBS, workspace=ws_d)

    def rel(o):
        return round(float((o - full).norm() / full.norm()), 4)
    errs = {}
    for name, sinks in [("recent_256", 0), ("sinks_4_recent", 4)]:
        idx = np.full((C, Hkv, budget), -1, dtype=np.int32)
        cnt = np.zeros((C, Hkv), dtype=np.int32)
        for i, p in enumerate(pos):
            lst = np.array(sorted(set(range(min(sinks, p + 1))) | set(range(max(0, p + 1 - (budget - sinks)), p + 1))))
            idx[i, :, :len(lst)] = lst
            cnt[i] = len(lst)
        o = torch.empty_like(full)
        K.sparse_attn(kvl, ql, Hq, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), budget, scale, o,
                      workspace=ws_s)
        errs[name] = rel(o)
    # Quest: summaries once, 16 pages of 16 per query head
    summary = torch.empty((n_pages, Hkv, 2, d), dtype=torch.bfloat16, device="cuda")
    K.quest_summarize(K.PagedKV(kp, vp, bt.cuda(), torch.tensor([N], dtype=torch.int32, device="cuda"), P, N), summary)
    qidx = torch.empty((C, Hq, 16 * P + P - 1), dtype=torch.int32, device="cuda")
    qcnt = torch.empty((C, Hq), dtype=torch.int32, device="cuda")
    ws_q = torch.empty(K.quest_workspace_bytes(kvl, Hq, 16), dtype=torch.uint8, device="cuda")
    ws_qs = torch.empty(K.sparse_workspace_bytes(C, Hq, d, qidx.shape[-1]), dtype=torch.uint8, device="cuda")
    oq = torch.empty_like(full)

    def quest():
        K.quest_select(kvl, summary, ql, Hq, 16, qidx, qcnt, workspace=ws_q)
        K.sparse_attn(kvl, ql, Hq, qidx, qcnt, qidx.shape[-1], scale, oq, workspace=ws_qs)
    t_quest = timed(torch, quest, 10)
    errs["quest_16_pages_per_prefix"] = rel(oq)
    # Quest as the experiment's code states it: pages ranked among all whole
    # pages of the prompt, then the positions after the query dropped
    kv_full = K.PagedKV(kp, vp, bt64, torch.full((C,), N, dtype=torch.int32, device="cuda"), P, N)
    qpos = torch.tensor(pos, dtype=torch.int32, device="cuda")
    oql = torch.empty_like(full)

    def quest_literal():
        K.quest_select_causal(kv_full, summary, ql, Hq, 16, qpos, qidx, qcnt, workspace=ws_q)
        K.sparse_attn(kv_full, ql, Hq, qidx, qcnt, qidx.shape[-1], scale, oql, workspace=ws_qs)
    t_quest_lit = timed(torch, quest_literal, 10)
    errs["quest_16_pages_whole_prompt_then_causal"] = rel(oql)
    # exact top-256 per query head
    logits = torch.empty((C, Hq, N), device="cuda")
    tk = torch.empty((C * Hq, budget), dtype=torch.int32, device="cuda")
    tc = torch.empty((C * Hq,), dtype=torch.int32, device="cuda")
    rl = kvl.seq_lens.repeat_interleave(Hq).to(torch.int32)
    ot = torch.empty_like(full)
    ws_t = torch.empty(K.sparse_workspace_bytes(C, Hq, d, budget), dtype=torch.uint8, device="cuda")

    def exact():
        K.decode_attn_scores(kvl, ql, Hq, scale, None, None, logits, K.EMIT_LOGITS, workspace=ws_d)
        K.select_keep(logits.view(C * Hq, N), rl, N, 0, 0, None, budget, tk, tc)
        K.sparse_attn(kvl, ql, Hq, tk.view(C, Hq, budget), tc.view(C, Hq), budget, scale, ot, workspace=ws_t)
    t_exact = timed(torch, exact, 10)
    errs["exact_top256"] = rel(ot)
    return {
        "metric": "KV GB/s (% HBM peak) for score-emitting decode attn + keep-set select",
        "value": round(kv_bytes / (t_all * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "qwen_like_chunks", "tokens": N, "chunk": C, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": d, "page_size": P, "budget": budget},
        "note": "megabyte-sized and launch-bound: the per-chunk times are the figures; the errors are of "
                "synthetic N(0,1) data, whose attention is far from sparse",
        "keep_all_us_per_chunk": round(t_all * 1e3, 1),
        "policy_us_per_chunk": policy_us,
        "last_64_queries": {"rel_error_vs_full": errs, "quest_us": round(t_quest * 1e3, 1),
                            "quest_whole_prompt_then_causal_us": round(t_quest_lit * 1e3, 1),
                            "exact_top256_us": round(t_exact * 1e3, 1),
                            "quest_readings": "per_prefix: pages ranked among the whole pages of each query's "
                                              "causal prefix (the decode reading); whole_prompt_then_causal: "
                                              "ranked among all whole pages of the prompt, then positions "
                                              "after the query dropped (the experiment's code)"},
    }


def llama3_h2o_workload(torch, K, synth, args) -> dict:
    """Llama-3-8B-shape layer, B=16, ragged L_b ~ U[8K, 32K], H2O with the
    eviction inside the decode loop: the lists of kept positions are seeded
    by one full score-emitting decode pass and the 20% keep set (sinks 4,
    window 512), then ``steps`` decode steps each append the new token,
    attend over the kept keys only, fold the probabilities into the list
    scores and cut every list back to its budget."""
    steps = args.steps
    cfg = synth.llama3_8b_layer(steps=steps + 1, device="cuda")
    kvt = cfg["kv"]
    Bq, HQq, HKVq = 16, 32, 8
    base = kvt.seq_lens.clone()
    cap = int(base.max()) + steps + 1
    kv0 = K.PagedKV(kvt.k_pages, kvt.v_pages, kvt.block_table, base, 16, cap)
    full = torch.zeros((Bq, HKVq, cap), device="cuda")
    out = torch.empty((Bq, HQq, 128), device="cuda")
    K.decode_attn_scores(kv0, cfg["q_steps"][0], HQq, cfg["scale"], out, None, None, K.EMIT_PROBS, full, 1.0)
    budgets = (base.double() * 0.2).floor().to(torch.int32).repeat_interleave(HKVq).contiguous()
    budget = int(budgets.max())
    rows = full.view(Bq * HKVq, cap)
    keep = torch.zeros((Bq * HKVq, budget), dtype=torch.int32, device="cuda")
    kc = torch.empty((Bq * HKVq,), dtype=torch.int32, device="cuda")
    K.select_keep(rows, base.repeat_interleave(HKVq).to(torch.int32), cap, 4, 512, budgets, budget, keep, kc)
    stride = -(-(budget + 1) // 16) * 16
    slots = torch.zeros((Bq, HKVq, stride), dtype=torch.int32, device="cuda")
    cum = torch.zeros((Bq, HKVq, stride), device="cuda")
    slots.view(-1, stride)[:, :budget] = keep
    valid = torch.arange(budget, device="cuda")[None, :] < kc[:, None]
    cum.view(-1, stride)[:, :budget] = torch.where(valid, torch.gather(rows, 1, keep.long()), 0.0)
    cnt = kc.view(Bq, HKVq).clone()
    kv_s = [K.PagedKV(kvt.k_pages, kvt.v_pages, kvt.block_table, (base + s + 1).to(torch.int32), 16, cap)
            for s in range(steps)]
    ws = torch.empty(K.h2o_workspace_bytes(kv0, HQq, stride, 4, 512, budget), dtype=torch.uint8, device="cuda")
    bview = budgets.view(Bq, HKVq)
    # untimed warm-up on copies of the lists
    s2, c2, n2 = slots.clone(), cum.clone(), cnt.clone()
    for s in range(2):
        K.h2o_step(kv_s[s], cfg["q_steps"][s + 1], HQq, cfg["scale"], s2, c2, n2, 4, 512, budget, out,
                   budgets=bview, workspace=ws)
    del s2, c2, n2
    torch.cuda.synchronize()
    kept_before = int(cnt.sum())
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for s in range(steps):
        K.h2o_step(kv_s[s], cfg["q_steps"][s + 1], HQq, cfg["scale"], slots, cum, cnt, 4, 512, budget, out,
                   budgets=bview, workspace=ws)
    b.record()
    torch.cuda.synchronize()
    t = a.elapsed_time(b) / steps
    kept_after = int(cnt.sum())
    # keys read per step: the kept lists plus the appended token
    keys = (kept_before + kept_after) / 2.0 + Bq * HKVq
    kv_bytes = keys * 128 * 2 * 2
    full_keys = float(base.sum()) * HKVq
    return {
        "metric": "KV GB/s (% HBM peak) for score-emitting decode attn + keep-set select",
        "value": round(kv_bytes / (t * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama3_8b_h2o_evict", "batch": Bq, "seq_len": "U[8192,32768]", "q_heads": HQq,
                   "kv_heads": HKVq, "head_dim": 128, "page_size": 16,
                   "keep": "0.2 L per sequence (sinks 4, window 512), evicted every step"},
        "step_us": round(t * 1e3, 1),
        "kept_keys_per_step": round(keys),
        "kept_fraction": round(keys / full_keys, 4),
        "launches_per_step": 2,
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; the Llama-3-8B workload runs its stated 256 decode steps, "
                         "the 128K workload its 64 sparse decode steps)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay each part of the step as a captured HIP graph (measured slower than "
                         "eager launches on this path)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--workload", default="llama70b_step",
                    choices=["llama70b_step", "long_context_128k", "llama3_8b_steps", "llama3_8b_h2o_evict",
                             "qwen_like_chunks", "tiny_case"],
                    help="the default is the 70B decode step; the others report their own line")
    ap.add_argument("--counters", action="store_true",
                    help="counter-collection mode: one layer, 3 decode calls, then a plain 1 GiB "
                         "device copy used to calibrate FETCH_SIZE / WRITE_SIZE (with --workload "
                         "long_context_128k: three SnapKV votes); prints no JSON")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = {"llama3_8b_steps": 256, "long_context_128k": 64}.get(args.workload, 20)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this path has no "
              "multi-GPU component to run", file=sys.stderr)
        return 2

    import torch
    import attention_score_guided_amd as K
    import synth
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        return 2

    if args.counters and args.workload == "long_context_128k":
        long_context_workload(torch, K, synth, args)
        return 0
    if args.counters:
        return counters_mode(torch, K, synth)
    if args.workload == "long_context_128k":
        print(json.dumps(long_context_workload(torch, K, synth, args)), flush=True)
        return 0
    if args.workload == "llama3_8b_steps":
        print(json.dumps(llama3_workload(torch, K, synth, args)), flush=True)
        return 0
    if args.workload == "tiny_case":
        print(json.dumps(tiny_workload(torch, K, synth, args)), flush=True)
        return 0
    if args.workload == "qwen_like_chunks":
        print(json.dumps(qwen_like_workload(torch, K, synth, args)), flush=True)
        return 0
    if args.workload == "llama3_8b_h2o_evict":
        print(json.dumps(llama3_h2o_workload(torch, K, synth, args)), flush=True)
        return 0

    log("setup: generating 80 layers of synthetic paged KV on the GPU")
    t0 = time.time()
    layers, bufs = setup(torch, K, synth)
    torch.cuda.synchronize()
    log(f"setup done in {time.time() - t0:.1f} s")
    scale = 1.0 / math.sqrt(D)

    if not args.graph:
        run_decode = lambda: step_decode(K, layers, bufs, scale)  # noqa: E731
        run_select = lambda: step_select(K, layers, bufs)  # noqa: E731
    else:
        # Each part of the step is one graph: 160 (decode) and 5 (select)
        # kernel launches replayed without host round trips.
        g_dec = capture(torch, lambda: step_decode(K, layers, bufs, scale))
        g_sel = capture(torch, lambda: step_select(K, layers, bufs))
        run_decode, run_select = g_dec.replay, g_sel.replay

    for _ in range(args.warmup):
        run_decode()
        run_select()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record()
        run_decode()
        ev[i][1].record()
        run_select()
        ev[i][2].record()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    dec_ms = [e[0].elapsed_time(e[1]) for e in ev]
    sel_ms = [e[1].elapsed_time(e[2]) for e in ev]
    step_ms = sorted(e[0].elapsed_time(e[2]) for e in ev)
    ms_median = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else 0.5 * (step_ms[len(step_ms) // 2 - 1] +
                                                                           step_ms[len(step_ms) // 2])
    dec_avg_ms = sum(dec_ms) / len(dec_ms) / LAYERS
    sel_avg_ms = sum(sel_ms) / len(sel_ms)
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step (host wall {wall / args.steps * 1e3:.3f} ms), "
        f"decode call avg {dec_avg_ms * 1e3:.1f} us, aggregate+select {sel_avg_ms * 1e3:.1f} us/step")

    # sanity: one step's probability mass per sequence and layer equals H_q
    mass = float(bufs["cum"][0].double().sum()) / B / (args.steps + args.warmup)
    kept = int(bufs["keep_cnt"].sum())

    probe = read_probe(torch, K)
    kv_step = LAYERS * kv_bytes_per_layer()
    value = kv_step / (ms_step * 1e-3) / 1e9
    alg = decode_algorithmic_bytes()
    achieved = alg / (dec_avg_ms * 1e-3) / 1e9
    tr = traffic_entry()
    line = {
        "metric": "KV GB/s (% HBM peak) for score-emitting decode attn + keep-set select",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama70b_step", "layers": LAYERS, "batch": B, "seq_len": L,
                   "q_heads": HQ, "kv_heads": HKV, "head_dim": D, "page_size": PAGE,
                   "block_size": BLOCK, "budget_frac": BUDGET_FRAC, "probs_emitted": True,
                   "parallelism": "single_gpu"},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if tr is None else int(tr),
                     "kernel": "kvsel_decode_attn_scores_agg of one layer (decode_partial_mfma, which "
                               "also normalises the probabilities, folds cum and writes its block "
                               "max/mean, + decode_combine); HIP events around the 80 decode calls "
                               "of each step, divided by 80",
                     "algorithmic_bytes": alg, "avg_call_us": round(dec_avg_ms * 1e3, 2)},
        "extra": {"ms_per_step_median": round(ms_median, 4),
                  "timing": "value and ms_per_step: the K timed steps between two events (mean); "
                            "ms_per_step_median: the median of the per-step event intervals",
                  "decode_share_of_step": round(dec_avg_ms * LAYERS / ms_step, 4),
                  "aggregate_select_us_per_step": round(sel_avg_ms * 1e3, 2),
                  "launch": "hip_graph" if args.graph else "eager",
                  "prob_mass_per_seq_layer_step": round(mass, 4), "blocks_kept": kept,
                  "hbm_read_probe_gb_per_s": round(probe, 1),
                  "read_probe": "kvsel_read_probe over 4 GiB on the same GPU (16-byte streaming loads, "
                                "nothing written), after the timed region; context for the 8 TB/s peak, "
                                "not used in value or frac"},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline: timing the float64 oracle on a sample")
        line["cpu_baseline"] = cpu_baseline(torch, layers, scale, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
