"""Qwen3-0.6B-like layer at full size (16 / 8 heads, d=128, bf16, 1600
tokens in 64-token chunks, causal within each chunk), against the float64
oracle:
  * keep-all: every chunk query attends to all earlier keys (the decode pass
    with one pseudo-sequence per chunk query, lengths p + 1);
  * recent-256 and sinks-4 + recent window: after every chunk the cache is cut
    back to 256 keys by the keep-set selection (k = 0: the policy's forced
    sets), and the next chunk attends to the kept keys plus its own causal
    prefix (sparse attention over those positions);
  * exact top-256 per query on the last 64 queries: the decode pass in
    logits mode, the row selection, sparse attention;
  * Quest (16 pages of 16 per query head) on the last 64 queries.
Outputs within 2e-3 relative L2, keep sets bit-exact."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.parity_util import f64, note, rel_l2
from tests.test_gpu_quest import _check_row

pytestmark = pytest.mark.gpu
OUT_TOL = 2e-3


def _K():
    import attention_score_guided_amd as K
    return K


def _paged(cfg, P=16):
    g = synth.generator(21)
    K_, V_ = cfg["K"], cfg["V"]
    Hkv, N, d = K_.shape
    bt, n_pages = synth.shuffled_block_table(1, N, P, g)
    kp = torch.zeros((n_pages, Hkv, P, d), dtype=torch.bfloat16)
    vp = torch.zeros((n_pages, Hkv, P, d), dtype=torch.bfloat16)
    synth.write_positions(kp, bt[0], 0, K_.cpu())
    synth.write_positions(vp, bt[0], 0, V_.cpu())
    return kp.cuda(), vp.cuda(), bt


@pytest.mark.parametrize("policy", ["keep_all", "recent", "sinks_recent"])
def test_qwen_like_chunked_prefill_policies(policy):
    K = _K()
    note(f"qwen-like chunked prefill, policy {policy}")
    cfg = synth.qwen_like_layer()
    Kd, Vd, Qd = f64(cfg["K"]), f64(cfg["V"]), f64(cfg["Q"])
    Hkv, N, d = Kd.shape
    Hq, C, budget, scale = cfg["num_q_heads"], cfg["chunk"], cfg["budget"], cfg["scale"]
    kp, vp, bt = _paged(cfg)
    sinks = {"keep_all": 0, "recent": 0, "sinks_recent": 4}[policy]
    bt64 = bt.repeat(C, 1).cuda()                       # one pseudo-sequence per chunk query
    kept = np.arange(0)
    stride = budget + C
    for c0 in range(0, N, C):
        pos = np.arange(c0, c0 + C)
        q = cfg["Q"][:, c0:c0 + C].permute(1, 0, 2).contiguous().cuda()      # [C][Hq][d]
        out = torch.empty((C, Hq, d), device="cuda")
        if policy == "keep_all":
            lens = torch.tensor(pos + 1, dtype=torch.int32, device="cuda")
            kv = K.PagedKV(kp, vp, bt64, lens, 16, c0 + C)
            K.decode_attn_scores(kv, q, Hq, scale, out, None, None, K.EMIT_PROBS)
        else:
            idx = np.full((C, Hkv, stride), -1, dtype=np.int32)
            cnt = np.zeros((C, Hkv), dtype=np.int32)
            for i in range(C):
                lst = np.concatenate([kept, pos[:i + 1]])
                idx[i, :, :len(lst)] = lst
                cnt[i] = len(lst)
            lens = torch.full((C,), c0 + C, dtype=torch.int32, device="cuda")
            kv = K.PagedKV(kp, vp, bt64, lens, 16, c0 + C)
            K.sparse_attn(kv, q, Hq, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), stride, scale, out)
        torch.cuda.synchronize()
        cache = np.arange(c0) if policy == "keep_all" else kept
        want, _ = O.chunk_causal_attention(Qd[:, c0:c0 + C], Kd[:, cache], Vd[:, cache], Kd[:, pos], Vd[:, pos],
                                           scale)
        assert rel_l2(f64(out), want) < OUT_TOL, c0
        if policy != "keep_all":
            # cut back to the budget: the policy's forced sets over all positions so far
            L = c0 + C
            rows = torch.zeros((1, L), device="cuda")
            keep = torch.empty((1, budget), dtype=torch.int32, device="cuda")
            kc = torch.empty((1,), dtype=torch.int32, device="cuda")
            K.select_keep(rows, torch.tensor([L], dtype=torch.int32, device="cuda"), L, sinks, budget - sinks,
                          None, budget, keep, kc)
            torch.cuda.synchronize()
            got = keep[0, :int(kc[0])].cpu().numpy()
            want_keep = O.recent_keep(L, budget) if policy == "recent" else O.streaming_keep(L, budget, 4)
            assert got.tolist() == want_keep.tolist()
            kept = got.astype(np.int64)


def test_qwen_like_exact_top256_on_last_queries():
    K = _K()
    cfg = synth.qwen_like_layer()
    Kd, Vd, Qd = f64(cfg["K"]), f64(cfg["V"]), f64(cfg["Q"])
    Hkv, N, d = Kd.shape
    Hq, C, scale = cfg["num_q_heads"], 64, cfg["scale"]
    kp, vp, bt = _paged(cfg)
    pos = np.arange(N - C, N)
    lens = torch.tensor(pos + 1, dtype=torch.int32, device="cuda")
    kv = K.PagedKV(kp, vp, bt.repeat(C, 1).cuda(), lens, 16, N)
    q = cfg["Q"][:, N - C:].permute(1, 0, 2).contiguous().cuda()
    logits = torch.empty((C, Hq, N), device="cuda")
    K.decode_attn_scores(kv, q, Hq, scale, None, None, logits, K.EMIT_LOGITS)
    rows = logits.view(C * Hq, N)
    rl = lens.repeat_interleave(Hq).to(torch.int32)
    keep = torch.empty((C * Hq, 256), dtype=torch.int32, device="cuda")
    kc = torch.empty((C * Hq,), dtype=torch.int32, device="cuda")
    K.select_keep(rows, rl, N, 0, 0, None, 256, keep, kc)
    out = torch.empty((C, Hq, d), device="cuda")
    K.sparse_attn(kv, q, Hq, keep.view(C, Hq, 256), kc.view(C, Hq), 256, scale, out)
    torch.cuda.synchronize()
    lg = f64(logits)
    for i in range(0, C, 9):
        p = int(pos[i])
        want_logits = scale * np.einsum("hd,hjd->hj", Qd[:, p], np.repeat(Kd[:, :p + 1], Hq // Hkv, axis=0))
        assert np.max(np.abs(lg[i, :, :p + 1] - want_logits)) < 1e-4 * np.abs(want_logits).max()
        sets = []
        for h in range(Hq):
            s = O.select_keep(lg[i, h], p + 1, 0, 0, 256)
            assert keep[i * Hq + h, :int(kc[i * Hq + h])].cpu().numpy().tolist() == s.tolist()
            sets.append(s)
        want, _ = O.sparse_attention(Qd[:, p], Kd, Vd, sets, scale)
        assert rel_l2(f64(out[i]), want) < OUT_TOL


def test_qwen_like_quest_on_last_queries():
    """The Quest strategy of the same experiment: page summaries (16 tokens)
    once over the prompt, then for each of the last 64 queries the 16 pages
    with the largest bounds over its causal prefix (plus the partial tail
    page), and sparse attention over them; sets and outputs against the
    oracle."""
    K = _K()
    cfg = synth.qwen_like_layer()
    Kd, Vd, Qd = f64(cfg["K"]), f64(cfg["V"]), f64(cfg["Q"])
    Hkv, N, d = Kd.shape
    Hq, C, scale, P = cfg["num_q_heads"], 64, cfg["scale"], 16
    G = Hq // Hkv
    kp, vp, bt = _paged(cfg)
    full = K.PagedKV(kp, vp, bt.cuda(), torch.tensor([N], dtype=torch.int32, device="cuda"), P, N)
    summary = torch.empty((kp.shape[0], Hkv, 2, d), dtype=torch.bfloat16, device="cuda")
    K.quest_summarize(full, summary)
    pos = np.arange(N - C, N)
    kv = K.PagedKV(kp, vp, bt.repeat(C, 1).cuda(), torch.tensor(pos + 1, dtype=torch.int32, device="cuda"), P, N)
    q = cfg["Q"][:, N - C:].permute(1, 0, 2).contiguous().cuda()
    idx = torch.empty((C, Hq, 16 * P + P - 1), dtype=torch.int32, device="cuda")
    cnt = torch.empty((C, Hq), dtype=torch.int32, device="cuda")
    bounds = torch.empty((C, Hq, N // P), device="cuda")
    K.quest_select(kv, summary, q, Hq, 16, idx, cnt, bounds=bounds)
    out = torch.empty((C, Hq, d), device="cuda")
    K.sparse_attn(kv, q, Hq, idx, cnt, idx.shape[-1], scale, out)
    torch.cuda.synchronize()
    for i in range(0, C, 7):
        p = int(pos[i])
        sets = []
        for h in range(Hq):
            got = idx[i, h, :int(cnt[i, h])].cpu().numpy()
            # the oracle's pages, except swaps between bounds within rounding of the cut
            _check_row(Qd[h, p], Kd[h // G, :p + 1], P, 16, f64(bounds[i, h]), got)
            sets.append(got)
        o_out, _ = O.sparse_attention(Qd[:, p], Kd, Vd, sets, scale)
        assert rel_l2(f64(out[i]), o_out) < OUT_TOL


def test_qwen_like_quest_literal_reading_on_last_queries():
    """The Quest cell of the experiment as its code states it: the 16 pages
    are ranked among ALL whole pages of the 1600-token prompt (summaries of
    the whole prompt), and only then are positions after the query dropped
    (kvsel_quest_select_causal).  Sets against oracle.quest_page_selection on
    the full keys: any difference must be a page whose bound lies within
    rounding of the 16th bound.  Outputs against the oracle's sparse
    attention on the GPU's sets."""
    K = _K()
    cfg = synth.qwen_like_layer()
    Kd, Vd, Qd = f64(cfg["K"]), f64(cfg["V"]), f64(cfg["Q"])
    Hkv, N, d = Kd.shape
    Hq, C, scale, P, budget = cfg["num_q_heads"], 64, cfg["scale"], 16, 16
    G = Hq // Hkv
    kp, vp, bt = _paged(cfg)
    full = K.PagedKV(kp, vp, bt.cuda(), torch.tensor([N], dtype=torch.int32, device="cuda"), P, N)
    summary = torch.empty((kp.shape[0], Hkv, 2, d), dtype=torch.bfloat16, device="cuda")
    K.quest_summarize(full, summary)
    pos = np.arange(N - C, N)
    kv = K.PagedKV(kp, vp, bt.repeat(C, 1).cuda(), torch.full((C,), N, dtype=torch.int32, device="cuda"), P, N)
    qpos = torch.tensor(pos, dtype=torch.int32, device="cuda")
    q = cfg["Q"][:, N - C:].permute(1, 0, 2).contiguous().cuda()
    idx = torch.full((C, Hq, budget * P + P - 1), -7, dtype=torch.int32, device="cuda")
    cnt = torch.empty((C, Hq), dtype=torch.int32, device="cuda")
    bounds = torch.empty((C, Hq, N // P), device="cuda")
    K.quest_select_causal(kv, summary, q, Hq, budget, qpos, idx, cnt, bounds=bounds)
    out = torch.empty((C, Hq, d), device="cuda")
    K.sparse_attn(kv, q, Hq, idx, cnt, idx.shape[-1], scale, out)
    torch.cuda.synchronize()
    from tests.test_gpu_quest import BOUND_TOL
    worst = 0.0
    for i in range(0, C, 3):
        p = int(pos[i])
        sets = []
        for h in range(Hq):
            Kh = Kd[h // G]
            got = idx[i, h, :int(cnt[i, h])].cpu().numpy()
            assert (idx[i, h, int(cnt[i, h]):] == -7).all()
            assert np.all(np.diff(got) > 0) and got.max() <= p
            kmin, kmax = O.quest_page_summary(Kh, P)
            want_b = O.quest_page_bounds(Qd[h, p], kmin, kmax)
            tol = BOUND_TOL * (np.abs(Qd[h, p]) * np.maximum(np.abs(kmin), np.abs(kmax))).sum(axis=1).max()
            assert np.max(np.abs(f64(bounds[i, h]) - want_b)) <= tol
            want = O.quest_page_selection(Qd[h, p], Kh, p, budget * P, P)
            if got.tolist() != want.tolist():
                kth = np.sort(want_b)[::-1][budget - 1]
                gs, ws_ = set(got.tolist()), set(want.tolist())
                for pg in sorted({j // P for j in gs ^ ws_}):
                    assert abs(want_b[pg] - kth) <= 2 * tol, (i, h, pg, want_b[pg], kth)
                    worst = max(worst, abs(want_b[pg] - kth) / tol)
            sets.append(got)
        o_out, _ = O.sparse_attention(Qd[:, p], Kd, Vd, sets, scale)
        assert rel_l2(f64(out[i]), o_out) < OUT_TOL
    note(f"literal Quest: page swaps at most {worst:.2f} of the bound tolerance from the cut")
