"""The hot-path calls captured in a HIP graph (as bench.py replays them)
give, on every replay, bit-identical results to the same calls run eagerly.
Between replays the test does eager work of its own (resetting the scores)
and synchronises."""
import math

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    import attention_score_guided_amd as K
    layers_n, B, Hq, Hkv, d, L, P, BS = 2, 2, 16, 2, 128, 4096, 64, 64
    g = synth.generator(77)
    bt, n_pages = synth.shuffled_block_table(B, L, P, g)
    lens = torch.tensor([L, 3000], dtype=torch.int32).cuda()
    layers = []
    for _ in range(layers_n):
        kp = synth.normal((n_pages, Hkv, P, d), g, torch.bfloat16).cuda()
        vp = synth.normal((n_pages, Hkv, P, d), g, torch.bfloat16).cuda()
        q = synth.normal((B, Hq, d), g, torch.bfloat16).cuda()
        layers.append((K.PagedKV(kp, vp, bt.cuda(), lens, P, L), q))
    scale = 1 / math.sqrt(d)
    n_blk = L // BS
    out = torch.empty((B, Hq, d), device="cuda")
    probs = torch.empty((B, Hq, L), device="cuda")
    cum = torch.zeros((layers_n, B, Hkv, L), device="cuda")
    agg = torch.zeros((B, n_blk), device="cuda")
    blk_lens = ((lens + BS - 1) // BS).to(torch.int32)
    idx = torch.empty((B, n_blk), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B,), dtype=torch.int32, device="cuda")
    ws = torch.empty(K.decode_workspace_bytes(layers[0][0], Hq, True), dtype=torch.uint8, device="cuda")
    ws_sel = torch.empty(K.select_workspace_bytes(B, n_blk, K.SELECT_GLOBAL_PERCENTILE), dtype=torch.uint8,
                         device="cuda")

    def step():
        for li, (kv, q) in enumerate(layers):
            K.decode_attn_scores(kv, q, Hq, scale, out, None, probs, K.EMIT_PROBS, cum[li], 1.0, workspace=ws)
        for li in range(layers_n):
            K.block_aggregate(cum[li], lens, L, BS, K.REDUCE_SUM, li > 0, agg, None)
        K.select_keep(agg, blk_lens, n_blk, 0, 0, None, 0, idx, cnt, mode=K.SELECT_GLOBAL_PERCENTILE,
                      global_budget=n_blk // 2, workspace=ws_sel)

    def snapshot():
        return [t.clone() for t in (out, probs, cum, agg, idx, cnt)]

    step()
    torch.cuda.synchronize()
    eager = snapshot()

    cum.zero_()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        cum.zero_()                 # the test's own eager work between replays
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(snapshot(), eager):
            assert torch.equal(a, b), f"replay {rep} differs from the eager run"
