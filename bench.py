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
    (probabilities emitted, cumulative scores updated)."""
    for li, (kv, q) in enumerate(layers):
        K.decode_attn_scores(kv, q, HQ, scale, bufs["out"], bufs["lse"], bufs["probs"], K.EMIT_PROBS,
                             bufs["cum"][li], 1.0, workspace=bufs["ws_dec"])


def step_select(K, layers, bufs):
    """Part 2 of a step: block aggregation summed over heads and layers, then
    the per-request percentile and the global top-K of blocks."""
    n_blk = L // BLOCK
    for li in range(len(layers)):
        K.block_aggregate(bufs["cum"][li], bufs["lens"], L, BLOCK, K.REDUCE_SUM, li > 0,
                          bufs["agg_max"], bufs["agg_mean"])
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
    return {"value": round(bytes_done / t_total / 1e9, 4), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{rows} (layer, sequence, KV head) rows from the first layers ({rows * 8} query "
                      f"heads x {L} keys; {rows / 64:.2f} of 80 layers): page gather, bf16 widening, "
                      f"attention, accumulation, block max/mean; {t_total:.1f} s"}


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
        kv, q = layers[0]
        K.decode_attn_scores(kv, q, HQ, scale, bufs["out"], bufs["lse"], bufs["probs"], K.EMIT_PROBS,
                             bufs["cum"][0], 1.0, workspace=bufs["ws_dec"])
    torch.cuda.synchronize()
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    log("counters mode done: decode x3, copy of 1073741824 bytes")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay each part of the step as a captured HIP graph (measured slower than "
                         "eager launches on this path)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--counters", action="store_true",
                    help="counter-collection mode: one layer, 3 decode calls, then a plain 1 GiB "
                         "device copy used to calibrate FETCH_SIZE / WRITE_SIZE; prints no JSON")
    args = ap.parse_args()
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

    if args.counters:
        return counters_mode(torch, K, synth)

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
        # Each part of the step is one graph: 240 (decode) and 81 (select)
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
    dec_avg_ms = sum(dec_ms) / len(dec_ms) / LAYERS
    sel_avg_ms = sum(sel_ms) / len(sel_ms)
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step (host wall {wall / args.steps * 1e3:.3f} ms), "
        f"decode call avg {dec_avg_ms * 1e3:.1f} us, aggregate+select {sel_avg_ms * 1e3:.1f} us/step")

    # sanity: one step's probability mass per sequence and layer equals H_q
    mass = float(bufs["cum"][0].double().sum()) / B / (args.steps + args.warmup)
    kept = int(bufs["keep_cnt"].sum())

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
                     "kernel": "kvsel_decode_attn_scores of one layer (decode_partial_mfma + "
                               "decode_combine + decode_finalize); HIP events around the 80 decode "
                               "calls of each step, divided by 80",
                     "algorithmic_bytes": alg, "avg_call_us": round(dec_avg_ms * 1e3, 2)},
        "extra": {"decode_share_of_step": round(dec_avg_ms * LAYERS / ms_step, 4),
                  "aggregate_select_us_per_step": round(sel_avg_ms * 1e3, 2),
                  "launch": "hip_graph" if args.graph else "eager",
                  "prob_mass_per_seq_layer_step": round(mass, 4), "blocks_kept": kept},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline: timing the float64 oracle on a sample")
        line["cpu_baseline"] = cpu_baseline(torch, layers, scale, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
