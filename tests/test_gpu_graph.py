"""The hot-path calls captured in a HIP graph (as bench.py replays them)
give, on every replay, bit-identical results to the same calls run eagerly,
and a single decode call replayed with new inputs matches the oracle on every
replay.  Between replays the tests do eager work of their own and
synchronise."""
import math

import numpy as np
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
    # zero-filled: positions past a sequence's length are left untouched, and
    # uninitialised memory there may hold NaNs, which never compare equal
    probs = torch.zeros((B, Hq, L), device="cuda")
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


def _valid_post_pairs(ws: torch.Tensor) -> int:
    """Number of 16-byte-aligned word pairs in a workspace that would pass the
    decode pass's post check under SOME tag: (tag << 32 | v, ~tag << 32 | v)
    with tag != 0.  Layout-free: it scans the whole buffer."""
    w = ws.cpu().numpy().view(np.uint64).reshape(-1, 2)
    hi0, hi1 = w[:, 0] >> np.uint64(32), w[:, 1] >> np.uint64(32)
    lo0, lo1 = w[:, 0] & np.uint64(0xFFFFFFFF), w[:, 1] & np.uint64(0xFFFFFFFF)
    ok = (hi0 != 0) & (hi1 == (hi0 ^ np.uint64(0xFFFFFFFF))) & (lo0 == lo1)
    return int(ok.sum())


def _probs_case(seed, B, Hkv, G, d, P, cap):
    g = synth.generator(seed)
    bt, n_pages = synth.shuffled_block_table(B, cap, P, g)
    kp = synth.normal((n_pages, Hkv, P, d), g, torch.bfloat16).cuda()
    vp = synth.normal((n_pages, Hkv, P, d), g, torch.bfloat16).cuda()
    return g, bt.cuda(), kp, vp


def test_no_post_survives_a_call():
    """After a decode call that normalises in-kernel, no word pair anywhere in
    its workspace validates as a post for any tag (the combine zeroes the
    pass's posts), so a later execution replaying the same tag cannot take a
    stale one.  The workspace starts as junk, as a fresh allocation might."""
    import attention_score_guided_amd as K
    B, Hkv, G, d, P, cap = 4, 4, 8, 128, 64, 8192
    Hq = Hkv * G
    g, bt, kp, vp = _probs_case(5, B, Hkv, G, d, P, cap)
    lens = torch.tensor([8192, 5000, 1, 7777], dtype=torch.int32).cuda()
    kv = K.PagedKV(kp, vp, bt, lens, P, cap)
    q = synth.normal((B, Hq, d), g, torch.bfloat16).cuda()
    nbytes = K.decode_workspace_bytes(kv, Hq, True)
    ws = torch.randint(0, 256, (nbytes // 16 * 16,), dtype=torch.uint8, device="cuda",
                       generator=torch.Generator(device="cuda").manual_seed(3))
    assert _valid_post_pairs(ws) == 0     # random junk: a chance pair is 2^-64 per pair
    out = torch.empty((B, Hq, d), device="cuda")
    probs = torch.empty((B, Hq, cap), device="cuda")
    cum = torch.zeros((B, Hkv, cap), device="cuda")
    for _ in range(2):
        K.decode_attn_scores(kv, q, Hq, 1 / math.sqrt(d), out, None, probs, K.EMIT_PROBS, cum, 1.0,
                             workspace=ws)
        torch.cuda.synchronize()
        n = _valid_post_pairs(ws)
        print(f"valid post pairs left in the workspace: {n}", flush=True)
        assert n == 0


def test_single_call_graph_replays_with_new_inputs():
    """One decode call (probabilities, cum, out) captured alone in a graph on
    its own workspace, replayed three times with a new query and longer
    device-side lengths written between replays.  Every replay is compared
    with the float64 oracle: probabilities and cum within 1e-4 relative, out
    within 2e-3 relative L2.  The grid (8 sequences x 8 KV heads x 16 chunks)
    exceeds the chip's resident workgroups, so rows meet at different times."""
    import attention_score_guided_amd as K
    import oracle as O
    from tests.parity_util import f64, logical_kv_rows, max_rel, rel_l2
    B, Hkv, G, d, P, cap = 8, 8, 8, 128, 64, 16384
    Hq = Hkv * G
    scale = 1 / math.sqrt(d)
    g, bt, kp, vp = _probs_case(6, B, Hkv, G, d, P, cap)
    lens0 = torch.randint(8192, 12000, (B,), generator=g, dtype=torch.int32)
    lens = lens0.cuda()
    kv = K.PagedKV(kp, vp, bt, lens, P, cap)
    q = torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((B, Hq, d), device="cuda")
    probs = torch.empty((B, Hq, cap), device="cuda")
    cum = torch.zeros((B, Hkv, cap), device="cuda")
    ws = torch.empty(K.decode_workspace_bytes(kv, Hq, True), dtype=torch.uint8, device="cuda")
    q.copy_(synth.normal((B, Hq, d), g, torch.bfloat16).cuda())
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            K.decode_attn_scores(kv, q, Hq, scale, out, None, probs, K.EMIT_PROBS, cum, 1.0, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    cum.zero_()
    cum_ref = np.zeros((B, Hkv, cap))
    cur = lens0.clone()
    for rep in range(3):
        if rep > 0:
            cur = torch.minimum(cur + torch.randint(1, 1500, (B,), generator=g, dtype=torch.int32),
                                torch.tensor(cap, dtype=torch.int32))
            q.copy_(synth.normal((B, Hq, d), g, torch.bfloat16).cuda())
            lens.copy_(cur.cuda())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        worst = [0.0, 0.0, 0.0]
        for b in range(B):
            L = int(cur[b])
            for c in range(Hkv):
                Kl, Vl = logical_kv_rows(kp, vp, bt, b, c, L)
                hs = slice(c * G, (c + 1) * G)
                r = O.decode_attention(f64(q[b, hs]), Kl, Vl, scale)
                cum_ref[b, c, :L] = O.accumulate(cum_ref[b, c:c + 1, :L], r["probs"])[0]
                e = (rel_l2(f64(out[b, hs]), r["out"]), max_rel(f64(probs[b, hs, :L]), r["probs"]),
                     max_rel(f64(cum[b, c, :L]), cum_ref[b, c, :L]))
                worst = [max(x, y) for x, y in zip(worst, e)]
                assert e[0] < 2e-3 and e[1] < 1e-4 and e[2] < 1e-4, (rep, b, c, e)
        print(f"replay {rep}: lengths {cur.tolist()} worst out {worst[0]:.2e} probs {worst[1]:.2e} "
              f"cum {worst[2]:.2e}", flush=True)


def test_sparse_step_graph_replays_with_new_queries():
    """One sparse decode step (indexer logits, the split top-2048 selection,
    sparse attention over the kept keys) captured in one graph, as bench.py
    replays it, and replayed with new queries copied into the captured inputs
    between replays: every replay equals the same step run eagerly on those
    queries, bit for bit (the path keeps no state between calls and clears
    nothing with memsets)."""
    import attention_score_guided_amd as K
    B, Hq, Hkv, d, dI, P, L, k = 2, 8, 2, 128, 64, 16, 40000, 2048
    g = synth.generator(91)
    bt, n_pages = synth.shuffled_block_table(B, L, P, g)
    bt = bt.cuda()
    kp = synth.normal((n_pages, Hkv, P, d), g, torch.bfloat16).cuda()
    vp = synth.normal((n_pages, Hkv, P, d), g, torch.bfloat16).cuda()
    kip = synth.normal((n_pages, 1, P, dI), g, torch.bfloat16).cuda()
    lens = torch.tensor([L, L - 777], dtype=torch.int32).cuda()
    kvi = K.PagedKV(kip, None, bt, lens, P, L)
    kvf = K.PagedKV(kp, vp, bt, lens, P, L)
    qi = torch.empty((B, Hq, dI), dtype=torch.bfloat16, device="cuda")
    q = torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    scores = torch.zeros((B, Hq, L), device="cuda")
    rl = lens.repeat_interleave(Hq).to(torch.int32)
    keep = torch.zeros((B * Hq, k), dtype=torch.int32, device="cuda")
    kc = torch.zeros((B * Hq,), dtype=torch.int32, device="cuda")
    out = torch.zeros((B, Hq, d), device="cuda")
    ws_d = torch.empty(K.decode_workspace_bytes(kvi, Hq, True), dtype=torch.uint8, device="cuda")
    ws_k = torch.empty(K.select_workspace_bytes(B * Hq, L, K.SELECT_ROWS), dtype=torch.uint8, device="cuda")
    ws_s = torch.empty(K.sparse_workspace_bytes(B, Hq, d, k), dtype=torch.uint8, device="cuda")

    def step():
        K.decode_attn_scores(kvi, qi, Hq, 1.0, None, None, scores, K.EMIT_LOGITS, workspace=ws_d)
        K.select_keep(scores.view(B * Hq, L), rl, L, 0, 0, None, k, keep, kc, workspace=ws_k)
        K.sparse_attn(kvf, q, Hq, keep.view(B, Hq, k), kc.view(B, Hq), k, 1 / math.sqrt(d), out, workspace=ws_s)

    def new_queries(seed):
        gg = synth.generator(seed)
        qi.copy_(synth.normal((B, Hq, dI), gg, torch.bfloat16).cuda())
        q.copy_(synth.normal((B, Hq, d), gg, torch.bfloat16).cuda())
        torch.cuda.synchronize()

    new_queries(1)
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        new_queries(100 + rep)
        step()                      # eager on the same queries
        torch.cuda.synchronize()
        want = [t.clone() for t in (scores, keep, kc, out)]
        out.fill_(float("nan"))
        keep.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((scores, keep, kc, out), want):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
        assert int(kc.min()) == k


def test_fused_sparse_step_graph_replays_with_new_queries():
    """The sparse decode step as bench.py times it (kvsel_indexer_topk, whose
    scores are never stored, then sparse attention) captured in one graph and
    replayed with new queries copied in between: every replay equals the
    eager step on those queries bit for bit, and the keep sets equal those of
    the stored-scores path."""
    import attention_score_guided_amd as K
    B, Hq, Hkv, d, dI, P, L, k = 2, 8, 2, 128, 64, 16, 40000, 2048
    g = synth.generator(92)
    bt, n_pages = synth.shuffled_block_table(B, L, P, g)
    bt = bt.cuda()
    kp = synth.normal((n_pages, Hkv, P, d), g, torch.bfloat16).cuda()
    vp = synth.normal((n_pages, Hkv, P, d), g, torch.bfloat16).cuda()
    kip = synth.normal((n_pages, 1, P, dI), g, torch.bfloat16).cuda()
    lens = torch.tensor([L, L - 777], dtype=torch.int32).cuda()
    kvi = K.PagedKV(kip, None, bt, lens, P, L)
    kvf = K.PagedKV(kp, vp, bt, lens, P, L)
    qi = torch.empty((B, Hq, dI), dtype=torch.bfloat16, device="cuda")
    q = torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    keep = torch.zeros((B * Hq, k), dtype=torch.int32, device="cuda")
    kc = torch.zeros((B * Hq,), dtype=torch.int32, device="cuda")
    out = torch.zeros((B, Hq, d), device="cuda")
    ws_x = torch.empty(K.indexer_topk_workspace_bytes(kvi, Hq, k), dtype=torch.uint8, device="cuda")
    ws_s = torch.empty(K.sparse_workspace_bytes(B, Hq, d, k), dtype=torch.uint8, device="cuda")
    scores = torch.zeros((B, Hq, L), device="cuda")
    rl = lens.repeat_interleave(Hq).to(torch.int32)
    keep_s = torch.zeros_like(keep)
    kc_s = torch.zeros_like(kc)

    def step():
        K.indexer_topk(kvi, qi, Hq, 1.0, k, keep, kc, workspace=ws_x)
        K.sparse_attn(kvf, q, Hq, keep.view(B, Hq, k), kc.view(B, Hq), k, 1 / math.sqrt(d), out, workspace=ws_s)

    def new_queries(seed):
        gg = synth.generator(seed)
        qi.copy_(synth.normal((B, Hq, dI), gg, torch.bfloat16).cuda())
        q.copy_(synth.normal((B, Hq, d), gg, torch.bfloat16).cuda())
        torch.cuda.synchronize()

    new_queries(1)
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        new_queries(200 + rep)
        step()                      # eager on the same queries
        K.decode_attn_scores(kvi, qi, Hq, 1.0, None, None, scores, K.EMIT_LOGITS)
        K.select_keep(scores.view(B * Hq, L), rl, L, 0, 0, None, k, keep_s, kc_s)
        torch.cuda.synchronize()
        assert torch.equal(keep, keep_s) and torch.equal(kc, kc_s), "fused keep sets differ from the stored-scores path"
        want = [t.clone() for t in (keep, kc, out)]
        out.fill_(float("nan"))
        keep.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((keep, kc, out), want):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
        assert int(kc.min()) == k


def test_h2o_step_graph_replays_with_new_tokens():
    """The H2O step with per-step eviction (two launches: the sparse pass
    that reads the current token as each list's next entry, and the tail
    kernel) captured once and replayed for successive tokens, with the
    sequence lengths and queries copied in between: after every replay the
    lists, their scores, their counts and the outputs equal those of eager
    steps run on a copy of the lists, bit for bit."""
    import attention_score_guided_amd as K
    B, Hq, Hkv, d, P, L0, T = 2, 8, 2, 128, 16, 3000, 4
    sinks, window, budget = 4, 64, 400
    g = synth.generator(93)
    cap = L0 + T + 1
    bt, n_pages = synth.shuffled_block_table(B, cap, P, g)
    bt = bt.cuda()
    kp = synth.normal((n_pages, Hkv, P, d), g, torch.bfloat16).cuda()
    vp = synth.normal((n_pages, Hkv, P, d), g, torch.bfloat16).cuda()
    qs = synth.normal((T, B, Hq, d), g, torch.bfloat16).cuda()
    stride = budget + 16
    # lists seeded with the last `budget` positions and random scores
    rng = torch.Generator().manual_seed(93)
    slots0 = torch.zeros((B, Hkv, stride), dtype=torch.int32)
    slots0[:, :, :budget] = torch.arange(L0 - budget, L0, dtype=torch.int32)
    cum0 = torch.zeros((B, Hkv, stride))
    cum0[:, :, :budget] = torch.rand((B, Hkv, budget), generator=rng)
    cnt0 = torch.full((B, Hkv), budget, dtype=torch.int32)
    slots0, cum0, cnt0 = slots0.cuda(), cum0.cuda(), cnt0.cuda()
    lens = torch.full((B,), L0 + 1, dtype=torch.int32, device="cuda")
    q = torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    kv = K.PagedKV(kp, vp, bt, lens, P, cap)
    scale = 1 / math.sqrt(d)

    def run(sl, cm, cn, out, ws):
        K.h2o_step(kv, q, Hq, scale, sl, cm, cn, sinks, window, budget, out, workspace=ws)

    ws_bytes = K.h2o_workspace_bytes(kv, Hq, stride, sinks, window, budget)
    g_state = [slots0.clone(), cum0.clone(), cnt0.clone(), torch.zeros((B, Hq, d), device="cuda"),
               torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")]
    e_state = [slots0.clone(), cum0.clone(), cnt0.clone(), torch.zeros((B, Hq, d), device="cuda"),
               torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")]
    q.copy_(qs[0])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    cap_state = [t.clone() for t in g_state[:3]]   # capture does not run the kernels
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            run(*g_state)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for t_, c_ in zip(g_state[:3], cap_state):
        t_.copy_(c_)
    for t in range(T):
        lens.fill_(L0 + 1 + t)
        q.copy_(qs[t])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        run(*e_state)
        torch.cuda.synchronize()
        n = e_state[2]
        assert torch.equal(g_state[2], n), f"replay {t}: counts differ"
        for b in range(B):
            for c in range(Hkv):
                m = int(n[b, c])
                assert torch.equal(g_state[0][b, c, :m], e_state[0][b, c, :m]), f"replay {t}: list ({b}, {c})"
                assert torch.equal(g_state[1][b, c, :m], e_state[1][b, c, :m]), f"replay {t}: scores ({b}, {c})"
        assert torch.equal(g_state[3], e_state[3]), f"replay {t}: outputs differ"
    assert int(g_state[2].min()) == budget   # one token in, one out per step
