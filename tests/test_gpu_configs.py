"""Each workload at its stated shape, in the launch configuration the
benchmark uses, end to end against the float64 oracle:
  * tiny case: 16 decode steps (fp32, probabilities emitted, cum fused), the
    block-16 max / mean and the keep set (sinks 4, window 64, budget 128);
  * Llama-3-8B-shape layer: all 256 decode steps at full size (B=16, ragged
    L_b ~ U[8K, 32K], cum fused, no probabilities), then block-16 max / mean
    and the 20% keep sets; sampled (sequence, KV head) rows in full after
    step 256, the probability mass of every row;
  * LLaMA-70B-shape step, two stacked layers at full size (B=8, L=32768, G=8,
    page 64): the fused decode + block-64 aggregation per layer, the head and
    layer sum at block size 1, and the global percentile top 25%; block
    scores of EVERY (layer, sequence, KV head) row and the kept blocks of
    every sequence;
  * 128K long-context case: all 64 sparse decode steps at full size (B=4,
    32 query heads, L = 131072 + s + 1), each step's indexer top-2048 by
    kvsel_indexer_topk (equal to the stored-scores path on every row of every
    step) and sparse attention; sampled rows of the first and last steps
    against the oracle (keep sets and attention outputs).
Keep sets are checked twice: bit-exact against the oracle's selection on the
GPU's own scores, and end to end against the oracle's selection on the
oracle's scores, where a difference must be a swap between scores within
1e-6 * max(1, |cut|) of the cut (the worst gap is printed)."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.parity_util import f64, keep_swap_gap, logical_kv, logical_kv_rows, max_rel, note, rel_l2

pytestmark = pytest.mark.gpu
OUT_TOL, SCORE_TOL = 2e-3, 1e-4


def _K():
    import attention_score_guided_amd as K
    return K


def test_tiny_case_end_to_end():
    K = _K()
    cfg = synth.tiny_case(device="cuda")
    kvt = cfg["kv"]
    prompt, steps, Hq, scale = cfg["prompt"], cfg["steps"], cfg["num_q_heads"], cfg["scale"]
    cap = prompt + steps
    kv_s = [K.PagedKV(kvt.k_pages, kvt.v_pages, kvt.block_table,
                      torch.tensor([prompt + s + 1], dtype=torch.int32, device="cuda"), 16, cap) for s in range(steps)]
    cum = torch.zeros((1, 1, cap), device="cuda")
    out = torch.empty((1, Hq, 64), device="cuda")
    probs = torch.empty((1, Hq, cap), device="cuda")
    ws = torch.empty(K.decode_workspace_bytes(kv_s[-1], Hq, True), dtype=torch.uint8, device="cuda")
    n_blk = cap // 16
    bmax = torch.empty((1, 1, n_blk), device="cuda")
    bmean = torch.empty((1, 1, n_blk), device="cuda")
    keep = torch.empty((1, 128), dtype=torch.int32, device="cuda")
    kc = torch.empty((1,), dtype=torch.int32, device="cuda")
    final = torch.tensor([cap], dtype=torch.int32, device="cuda")
    bud = torch.tensor([128], dtype=torch.int32, device="cuda")
    for s in range(steps):
        K.decode_attn_scores(kv_s[s], cfg["q_steps"][s], Hq, scale, out, None, probs, K.EMIT_PROBS, cum, 1.0,
                             workspace=ws)
    K.block_aggregate(cum, final, cap, 16, K.REDUCE_NONE, False, bmax, bmean)
    K.select_keep(cum.view(1, cap), final, cap, 4, 64, bud, 128, keep, kc)
    torch.cuda.synchronize()

    Kall, Vall = logical_kv(kvt.k_pages, kvt.v_pages, kvt.block_table, 0, cap)
    cum_ref = np.zeros((1, cap))
    for s in range(steps):
        L = prompt + s + 1
        r = O.decode_attention(f64(cfg["q_steps"][s, 0]), Kall[:, :L], Vall[:, :L], scale)
        cum_ref[:, :L] = O.accumulate(cum_ref[:, :L], r["probs"])
    assert rel_l2(f64(out[0]), r["out"]) < OUT_TOL                       # the last step's output
    assert max_rel(f64(probs[0]), r["probs"]) < SCORE_TOL                # and its probabilities
    assert max_rel(f64(cum[0]), cum_ref) < SCORE_TOL
    want_max, want_mean = O.block_aggregate(cum_ref, cap, 16)
    assert max_rel(f64(bmax[0]), want_max) < SCORE_TOL
    assert max_rel(f64(bmean[0]), want_mean) < SCORE_TOL
    got = keep[0, :int(kc[0])].cpu().numpy()
    assert got.tolist() == O.select_keep(f64(cum[0, 0]), cap, 4, 64, 128).tolist()
    e2e = O.select_keep(cum_ref[0], cap, 4, 64, 128)
    gap = keep_swap_gap(got, e2e, cum_ref[0], cap, 4, 64)
    note(f"tiny case keep set vs the oracle's: {len(set(got.tolist()) ^ set(e2e.tolist()))} differing, "
         f"worst gap {gap:.2e}")
    assert len(got) == 128 and got[:4].tolist() == [0, 1, 2, 3]


def test_llama3_8b_layer_256_steps_full_size_sampled():
    K = _K()
    steps = 256
    cfg = synth.llama3_8b_layer(steps=steps, device="cuda")
    kvt = cfg["kv"]
    B, Hq, Hkv, G = 16, 32, 8, 4
    base = kvt.seq_lens.clone()
    cap = int(base.max()) + steps
    stride = -(-cap // 16) * 16
    kv_s = [K.PagedKV(kvt.k_pages, kvt.v_pages, kvt.block_table, (base + s + 1).to(torch.int32), 16, cap)
            for s in range(steps)]
    cum = torch.zeros((B, Hkv, stride), device="cuda")
    out = torch.empty((B, Hq, 128), device="cuda")
    ws = torch.empty(K.decode_workspace_bytes(kv_s[0], Hq, False), dtype=torch.uint8, device="cuda")
    n_blk = -(-cap // 16)
    bmax = torch.zeros((B, Hkv, n_blk), device="cuda")
    bmean = torch.zeros((B, Hkv, n_blk), device="cuda")
    final = (base + steps).to(torch.int32)
    rl = final.repeat_interleave(Hkv).to(torch.int32)
    budgets = (rl.double() * 0.2).floor().to(torch.int32)
    mb = int(budgets.max())
    keep = torch.empty((B * Hkv, mb), dtype=torch.int32, device="cuda")
    kc = torch.empty((B * Hkv,), dtype=torch.int32, device="cuda")
    ws_sel = torch.empty(max(256, K.select_workspace_bytes(B * Hkv, cap, K.SELECT_ROWS)), dtype=torch.uint8,
                         device="cuda")
    for s in range(steps):
        K.decode_attn_scores(kv_s[s], cfg["q_steps"][s], Hq, cfg["scale"], out, None, None, K.EMIT_PROBS, cum, 1.0,
                             workspace=ws)
    K.block_aggregate(cum, final, cap, 16, K.REDUCE_NONE, False, bmax, bmean)
    K.select_keep(cum.view(B * Hkv, stride), rl, cap, 4, 512, budgets, mb, keep, kc, workspace=ws_sel)
    torch.cuda.synchronize()
    # every row: 256 steps x 4 query heads of probability mass
    sums = cum.double().sum(dim=2).cpu().numpy()
    np.testing.assert_allclose(sums, steps * G, rtol=1e-4)
    q_all = cfg["q_steps"].cpu()
    for b, c in [(3, 2), (12, 6)]:
        L = int(final[b])
        note(f"llama3 256-step row b={b} kvh={c} L={L}")
        Kl, _ = logical_kv_rows(kvt.k_pages, None, kvt.block_table, b, c, L)
        cum_ref = np.zeros((1, L))
        for s in range(steps):
            Ls = int(base[b]) + s + 1
            r = O.decode_attention(f64(q_all[s, b, c * G:(c + 1) * G]), Kl[:, :Ls], None, cfg["scale"])
            cum_ref[:, :Ls] = O.accumulate(cum_ref[:, :Ls], r["probs"])
        got = f64(cum[b, c, :L])
        assert max_rel(got, cum_ref[0]) < SCORE_TOL
        want_max, want_mean = O.block_aggregate(cum_ref, L, 16)
        nb = want_max.shape[1]
        assert max_rel(f64(bmax[b, c, :nb]), want_max[0]) < SCORE_TOL
        assert max_rel(f64(bmean[b, c, :nb]), want_mean[0]) < SCORE_TOL
        r_ = b * Hkv + c
        gk = keep[r_, :int(kc[r_])].cpu().numpy()
        assert gk.tolist() == O.select_keep(got, L, 4, 512, int(budgets[r_])).tolist()
        e2e = O.select_keep(cum_ref[0], L, 4, 512, int(budgets[r_]))
        gap = keep_swap_gap(gk, e2e, cum_ref[0], L, 4, 512)
        note(f"  20% keep set after 256 steps vs the oracle's: {len(set(gk.tolist()) ^ set(e2e.tolist()))} "
             f"differing, worst gap {gap:.2e}")


def test_llama70b_step_two_stacked_layers_full_size():
    K = _K()
    LAYERS, B, Hq, Hkv, G, L, P, BS = 2, 8, 64, 8, 8, 32768, 64, 64
    n_blk = L // BS
    bt, _ = synth.shuffled_block_table(B, L, P, synth.generator(4, "cuda"), "cuda")
    layers = []
    for li in range(LAYERS):
        cfg = synth.llama70b_layer(li, device="cuda", block_table=bt)
        kvt = cfg["kv"]
        layers.append((K.PagedKV(kvt.k_pages, kvt.v_pages, kvt.block_table, kvt.seq_lens, P, L), cfg["q"]))
    scale = 1 / math.sqrt(128)
    out = torch.empty((B, Hq, 128), device="cuda")
    lse = torch.empty((B, Hq), device="cuda")
    probs = torch.empty((B, Hq, L), device="cuda")
    cum = torch.zeros((LAYERS, B, Hkv, L), device="cuda")
    blk_max = torch.zeros((B, LAYERS * Hkv, n_blk), device="cuda")
    blk_mean = torch.zeros((B, LAYERS * Hkv, n_blk), device="cuda")
    agg_max = torch.zeros((B, n_blk), device="cuda")
    agg_mean = torch.zeros((B, n_blk), device="cuda")
    blk_lens = torch.full((B,), n_blk, dtype=torch.int32, device="cuda")
    keep_idx = torch.empty((B, n_blk), dtype=torch.int32, device="cuda")
    keep_cnt = torch.empty((B,), dtype=torch.int32, device="cuda")
    ws = torch.empty(K.decode_workspace_bytes(layers[0][0], Hq, True), dtype=torch.uint8, device="cuda")
    ws_sel = torch.empty(max(256, K.select_workspace_bytes(B, n_blk, K.SELECT_GLOBAL_PERCENTILE)),
                         dtype=torch.uint8, device="cuda")
    bm, bn = blk_max.view(-1), blk_mean.view(-1)
    for li, (kv, q) in enumerate(layers):
        off = li * Hkv * n_blk
        K.decode_attn_scores_agg(kv, q, Hq, scale, out, lse, probs, cum[li], 1.0, BS, bm[off:], bn[off:], n_blk,
                                 LAYERS * Hkv * n_blk, workspace=ws)
    K.block_aggregate(blk_max, blk_lens, n_blk, 1, K.REDUCE_SUM, False, agg_max, None)
    K.block_aggregate(blk_mean, blk_lens, n_blk, 1, K.REDUCE_SUM, False, agg_mean, None)
    budget = int(0.25 * B * n_blk)
    K.select_keep(agg_max, blk_lens, n_blk, 0, 0, None, 0, keep_idx, keep_cnt, mode=K.SELECT_GLOBAL_PERCENTILE,
                  global_budget=budget, workspace=ws_sel)
    torch.cuda.synchronize()

    want_agg_max = np.zeros((B, n_blk))
    want_agg_mean = np.zeros((B, n_blk))
    g_bmax, g_bmean = f64(blk_max), f64(blk_mean)
    for li, (kv, q) in enumerate(layers):
        for b in range(B):
            note(f"70B step layer {li} sequence {b}: 8 KV-head rows")
            for c in range(Hkv):
                Kl, _ = logical_kv_rows(kv.k_pages, None, kv.block_table, b, c, L)
                r = O.decode_attention(f64(q[b, c * G:(c + 1) * G]), Kl, None, scale)
                cum_ref = O.accumulate(np.zeros((1, L)), r["probs"])
                mx, mn = O.block_aggregate(cum_ref, L, BS)
                assert max_rel(g_bmax[b, li * Hkv + c], mx[0]) < SCORE_TOL, (li, b, c)
                assert max_rel(g_bmean[b, li * Hkv + c], mn[0]) < SCORE_TOL, (li, b, c)
                want_agg_max[b] += mx[0]
                want_agg_mean[b] += mn[0]
    assert max_rel(f64(agg_max), want_agg_max) < SCORE_TOL
    assert max_rel(f64(agg_mean), want_agg_mean) < SCORE_TOL
    lens = [n_blk] * B
    gsel = [keep_idx[b, :int(keep_cnt[b])].cpu().numpy() for b in range(B)]
    # the selection on the GPU's own block scores, bit-exact
    own = O.global_percentile_select([f64(agg_max[b]) for b in range(B)], lens, budget)
    for b in range(B):
        assert gsel[b].tolist() == list(own[b]), b
    # end to end: equal row lengths make the global percentile top 25% the
    # top quarter of every row, so each row is compared with the oracle's
    e2e = O.global_percentile_select([want_agg_max[b] for b in range(B)], lens, budget)
    worst = 0.0
    for b in range(B):
        worst = max(worst, keep_swap_gap(gsel[b], np.asarray(e2e[b]), want_agg_max[b], n_blk))
    assert sum(len(x) for x in gsel) == budget
    note(f"70B step kept blocks vs the oracle's: worst gap {worst:.2e}")


def test_long_context_128k_64_sparse_steps_full_size():
    K = _K()
    L, B, Hq, steps, k = 131072, 4, 32, 64, 2048
    cfg = synth.long_context_128k(seq_len=L, sparse_steps=steps, device="cuda")
    kvt, kit = cfg["kv"], cfg["kv_index"]
    cap = L + steps
    keep = torch.empty((B * Hq, k), dtype=torch.int32, device="cuda")
    kc = torch.empty((B * Hq,), dtype=torch.int32, device="cuda")
    keep_s = torch.empty_like(keep)
    kc_s = torch.empty_like(kc)
    scores = torch.empty((B, Hq, -(-cap // 64) * 64), device="cuda")
    out = torch.empty((B, Hq, 128), device="cuda")
    ws_x = torch.empty(K.indexer_topk_workspace_bytes(
        K.PagedKV(kit.k_pages, None, kit.block_table, kit.seq_lens, 16, cap), Hq, k), dtype=torch.uint8, device="cuda")
    checked = {}
    for s_ in range(steps):
        lens = torch.full((B,), L + s_ + 1, dtype=torch.int32, device="cuda")
        kvi = K.PagedKV(kit.k_pages, None, kit.block_table, lens, 16, cap)
        kvf = K.PagedKV(kvt.k_pages, kvt.v_pages, kvt.block_table, lens, 16, cap)
        K.indexer_topk(kvi, cfg["qi_dec"][s_], Hq, 1.0, k, keep, kc, workspace=ws_x)
        K.sparse_attn(kvf, cfg["q_dec"][s_], Hq, keep.view(B, Hq, k), kc.view(B, Hq), k, cfg["scale"], out)
        K.decode_attn_scores(kvi, cfg["qi_dec"][s_], Hq, 1.0, None, None, scores, K.EMIT_LOGITS)
        K.select_keep(scores.view(B * Hq, scores.shape[-1]), lens.repeat_interleave(Hq).to(torch.int32), cap, 0, 0,
                      None, k, keep_s, kc_s)
        torch.cuda.synchronize()
        assert torch.equal(kc, kc_s) and torch.equal(keep, keep_s), f"step {s_}: fused keep sets differ"
        assert int(kc.min()) == k
        if s_ in (0, steps - 1):
            checked[s_] = (keep.clone(), out.clone())
    for s_, (kk, oo) in checked.items():
        n = L + s_ + 1
        for b, h in [(0, 3), (3, 30)]:
            note(f"128K sparse step {s_ + 1}/{steps}, row b={b} h={h}")
            KI, _ = logical_kv_rows(kit.k_pages, None, kit.block_table, b, 0, n)
            want_s = O.indexer_scores(f64(cfg["qi_dec"][s_, b, h])[None, :], KI[0])[0]
            e2e = O.select_keep(want_s, n, 0, 0, k)
            got = kk[b * Hq + h].cpu().numpy()
            gap = keep_swap_gap(got, e2e, want_s, n)
            note(f"  top-2048 vs the oracle's: {len(set(got.tolist()) ^ set(e2e.tolist()))} differing, worst gap {gap:.2e}")
            Kl, Vl = logical_kv_rows(kvt.k_pages, kvt.v_pages, kvt.block_table, b, h // 4, n)
            so, _ = O.sparse_attention(f64(cfg["q_dec"][s_, b, h])[None, :], Kl, Vl, [np.sort(got)], cfg["scale"])
            assert rel_l2(f64(oo[b, h]), so[0]) < OUT_TOL
