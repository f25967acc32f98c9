"""GPU parity of kvsel_h2o_step (H2O with the eviction inside the decode
loop) against the float64 oracle, step by step: each GPU step is checked
against the oracle's step applied to the GPU's previous state (the slot
lists and scores), so a near-tie resolved differently cannot make later
steps diverge.  Outputs within 2e-3 relative L2, probabilities and scores
within 1e-4 relative, kept lists bit-exact except swaps between scores
within 1e-6 relative of the cut."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.parity_util import f64, logical_kv, max_rel, note, rel_l2

pytestmark = pytest.mark.gpu
OUT_TOL, SCORE_TOL, TIE_TOL = 2e-3, 1e-4, 1e-6


def _K():
    import attention_score_guided_amd as K
    return K


def _check_keep(got, want_lists, want_scores, folded, c_list):
    """got: kept positions; the oracle's kept positions and the folded
    scores of the appended list c_list.  Equal, or differing only by slots
    whose scores sit within TIE_TOL of the cut."""
    if got.tolist() == want_lists.tolist():
        return True
    kept_scores = folded[np.isin(c_list, want_lists)]
    cut = kept_scores.min()
    pos_score = dict(zip(c_list.tolist(), folded.tolist()))
    for pos in set(got.tolist()) ^ set(want_lists.tolist()):
        assert abs(pos_score[pos] - cut) <= TIE_TOL * max(abs(cut), 1e-30), (pos, pos_score[pos], cut)
    return False


def _check_step(q_b, Kl, Vl, L, prev, b, out_b, probs_b, slots, cum, cnt, G, scale, sinks, window, budget):
    """One sequence of one GPU step against the oracle's step from the GPU's
    previous state ``prev`` = (slots, scores, counts) as host arrays."""
    Hkv = prev[0].shape[1]
    kept = [prev[0][b, c, :prev[2][b, c]] for c in range(Hkv)]
    sc = [prev[1][b, c, :prev[2][b, c]] for c in range(Hkv)]
    o_out, o_probs, o_kept, o_cum = O.h2o_evict_step(q_b, Kl[:, :L], Vl[:, :L], kept, sc, scale, sinks, window,
                                                     budget)
    assert rel_l2(out_b, o_out) < OUT_TOL
    for c in range(Hkv):
        n_app = int(prev[2][b, c]) + 1
        if probs_b is not None:
            for h in range(c * G, (c + 1) * G):
                assert max_rel(probs_b[h, :n_app], o_probs[h]) < SCORE_TOL
                assert (probs_b[h, n_app:] == -9.0).all()
        c_list = np.append(kept[c], L - 1)
        folded = O.accumulate(np.append(sc[c], 0.0)[None, :], np.stack(o_probs[c * G:(c + 1) * G]))[0]
        n_new = int(cnt[b, c])
        assert n_new == len(o_kept[c])
        got = slots[b, c, :n_new]
        exact = _check_keep(got, o_kept[c], o_cum[c], folded, c_list)
        want_cum = np.array([folded[np.searchsorted(c_list, p)] for p in got])
        assert max_rel(cum[b, c, :n_new], want_cum) < SCORE_TOL
        if exact:
            assert max_rel(cum[b, c, :n_new], o_cum[c]) < SCORE_TOL


CASES = [
    # seed, dtype, d, G, Hkv, P, prompt lengths, steps, sinks, window, budget, slot_stride, probs
    (81, torch.bfloat16, 128, 4, 2, 16, [600, 150, 30], 24, 4, 16, 64, 80, True),
    (82, torch.float32, 64, 8, 1, 32, [300, 90], 16, 2, 8, 40, 41, False),
    (83, torch.bfloat16, 128, 1, 3, 16, [1000], 12, 4, 32, 300, 400, True),
    (84, torch.bfloat16, 64, 2, 2, 64, [2000, 500], 10, 0, 0, 100, 101, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}-d{c[2]}-G{c[3]}-k{c[10]}")
def test_h2o_step_against_oracle(case):
    seed, dtype, d, G, Hkv, P, prompts, T, sinks, window, budget, stride, want_probs = case
    note(f"h2o case {case}")
    K = _K()
    g = synth.generator(seed)
    B, Hq = len(prompts), Hkv * G
    cap = max(prompts) + T
    bt, n_pages = synth.shuffled_block_table(B, cap, P, g)
    kp = synth.normal((n_pages, Hkv, P, d), g, dtype).cuda()
    vp = synth.normal((n_pages, Hkv, P, d), g, dtype).cuda()
    qs = synth.normal((T, B, Hq, d), g, dtype).cuda()
    bt = bt.cuda()
    rng = np.random.default_rng(seed)
    # initial lists: the sinks plus a random ascending subset of the prompt,
    # with random seed scores (as a prefill vote would leave them)
    slots = torch.zeros((B, Hkv, stride), dtype=torch.int32)
    cum = torch.zeros((B, Hkv, stride))
    cnt = torch.zeros((B, Hkv), dtype=torch.int32)
    for b, L0 in enumerate(prompts):
        for c in range(Hkv):
            n0 = min(L0, budget)
            rest = np.sort(rng.choice(np.arange(min(sinks, L0), L0), n0 - min(sinks, L0), replace=False))
            lst = np.concatenate([np.arange(min(sinks, L0)), rest]).astype(np.int32)
            slots[b, c, :n0] = torch.from_numpy(lst)
            cum[b, c, :n0] = torch.from_numpy(rng.uniform(0, 3, n0).astype(np.float32))
            cnt[b, c] = n0
    slots, cum, cnt = slots.cuda(), cum.cuda(), cnt.cuda()
    scale = 1 / math.sqrt(d)
    logical = [logical_kv(kp, vp, bt, b, L0 + T) for b, L0 in enumerate(prompts)]
    lens0 = torch.tensor(prompts, dtype=torch.int32, device="cuda")
    ws = torch.empty(K.h2o_workspace_bytes(K.PagedKV(kp, vp, bt, lens0, P, cap), Hq, stride, sinks, window, budget),
                     dtype=torch.uint8, device="cuda")
    for t in range(T):
        lens = torch.tensor([L0 + t + 1 for L0 in prompts], dtype=torch.int32, device="cuda")
        kv = K.PagedKV(kp, vp, bt, lens, P, cap)
        prev = (f64(slots).astype(np.int64), f64(cum), cnt.cpu().numpy().copy())
        out = torch.empty((B, Hq, d), device="cuda")
        probs = torch.full((B, Hq, stride), -9.0, device="cuda") if want_probs else None
        K.h2o_step(kv, qs[t].contiguous(), Hq, scale, slots, cum, cnt, sinks, window, budget, out, probs,
                   workspace=ws)
        torch.cuda.synchronize()
        s_h, c_h, n_h, o_h = slots.cpu().numpy(), f64(cum), cnt.cpu().numpy(), f64(out)
        p_h = f64(probs) if want_probs else None
        for b, L0 in enumerate(prompts):
            Kl, Vl = logical[b]
            _check_step(f64(qs[t, b]), Kl, Vl, L0 + t + 1, prev, b, o_h[b], None if p_h is None else p_h[b],
                        s_h, c_h, n_h, G, scale, sinks, window, budget)


def test_h2o_step_llama3_shape_with_decode_seeded_lists():
    """Llama-3-8B-shape layer scaled down (B=4, 32 / 8 heads, L_b in [1000,
    3000]): lists seeded by one full score-emitting decode pass and the
    keep-set selection at 20% (sinks 4, window 64), then 6 steps of per-step
    eviction with the same per-sequence budgets; each step checked against
    the oracle on the GPU's state."""
    K = _K()
    steps = 6
    cfg = synth.llama3_8b_layer(num_seqs=4, min_len=1000, max_len=3000, steps=steps + 1, device="cuda")
    kvt = cfg["kv"]
    B, Hq, Hkv = 4, 32, 8
    base = kvt.seq_lens.clone()
    cap = int(base.max()) + steps + 1
    # seed: cum of one full decode step over the prompt, then the 20% keep set
    kv0 = K.PagedKV(kvt.k_pages, kvt.v_pages, kvt.block_table, base, 16, cap)
    full = torch.zeros((B, Hkv, cap), device="cuda")
    out = torch.empty((B, Hq, 128), device="cuda")
    K.decode_attn_scores(kv0, cfg["q_steps"][0], Hq, cfg["scale"], out, None, None, K.EMIT_PROBS, full, 1.0)
    budgets = (base.double() * 0.2).floor().to(torch.int32).repeat_interleave(Hkv)
    budget = int(budgets.max())
    rows = full.view(B * Hkv, cap)
    rl = base.repeat_interleave(Hkv).to(torch.int32)
    keep = torch.empty((B * Hkv, budget), dtype=torch.int32, device="cuda")
    kc = torch.empty((B * Hkv,), dtype=torch.int32, device="cuda")
    K.select_keep(rows, rl, cap, 4, 64, budgets, budget, keep, kc)
    stride = budget + 8
    slots = torch.zeros((B, Hkv, stride), dtype=torch.int32, device="cuda")
    cum = torch.zeros((B, Hkv, stride), device="cuda")
    slots.view(B * Hkv, stride)[:, :budget] = keep
    cum.view(B * Hkv, stride)[:, :budget] = torch.gather(rows, 1, keep.long().clamp(0, cap - 1))
    cnt = kc.view(B, Hkv).clone()
    torch.cuda.synchronize()
    for b in range(B):
        for c in range(Hkv):
            n = int(cnt[b, c])
            cum[b, c, n:] = 0
    logical = [logical_kv(kvt.k_pages, kvt.v_pages, kvt.block_table, b, int(base[b]) + steps + 1) for b in range(B)]
    for t in range(steps):
        lens = (base + t + 1).to(torch.int32)
        kv = K.PagedKV(kvt.k_pages, kvt.v_pages, kvt.block_table, lens, 16, cap)
        prev = (f64(slots).astype(np.int64), f64(cum), cnt.cpu().numpy().copy())
        q = cfg["q_steps"][t + 1].contiguous()
        K.h2o_step(kv, q, Hq, cfg["scale"], slots, cum, cnt, 4, 64, budget, out, budgets=budgets.view(B, Hkv))
        torch.cuda.synchronize()
        s_h, c_h, n_h, o_h = slots.cpu().numpy(), f64(cum), cnt.cpu().numpy(), f64(out)
        for b in range(B):
            Kl, Vl = logical[b]
            _check_step(f64(q[b]), Kl, Vl, int(lens[b]), prev, b, o_h[b], None, s_h, c_h, n_h, 4,
                        cfg["scale"], 4, 64, int(budgets[b * Hkv]))


def test_h2o_step_general_and_fused_eviction_paths():
    """A list seeded longer than its budget sheds many slots at the first
    step (the general selection) and one per step afterwards (the fused
    argmin); a list over 8192 slots always takes the general path.  Budgets
    differ per list (one below the forced sinks + window)."""
    K = _K()
    g = synth.generator(88)
    prompts, P, d, G, Hkv, T = [12000, 700], 16, 64, 2, 2, 3
    B, Hq = 2, Hkv * G
    cap = max(prompts) + T
    bt, n_pages = synth.shuffled_block_table(B, cap, P, g)
    kp = synth.normal((n_pages, Hkv, P, d), g, torch.bfloat16).cuda()
    vp = synth.normal((n_pages, Hkv, P, d), g, torch.bfloat16).cuda()
    qs = synth.normal((T, B, Hq, d), g, torch.bfloat16).cuda()
    bt = bt.cuda()
    stride = 12000 + T + 1
    slots = torch.zeros((B, Hkv, stride), dtype=torch.int32)
    cum = torch.zeros((B, Hkv, stride))
    cnt = torch.zeros((B, Hkv), dtype=torch.int32)
    rng = np.random.default_rng(88)
    for b, L0 in enumerate(prompts):
        for c in range(Hkv):
            slots[b, c, :L0] = torch.arange(L0, dtype=torch.int32)
            cum[b, c, :L0] = torch.from_numpy(rng.uniform(0, 3, L0).astype(np.float32))
            cnt[b, c] = L0
    slots, cum, cnt = slots.cuda(), cum.cuda(), cnt.cuda()
    # list (0, 0) keeps more than 8192 slots; (1, 1) has a budget below sinks + window
    budgets = torch.tensor([[10000, 3000], [500, 10]], dtype=torch.int32, device="cuda")
    scale = 1 / math.sqrt(d)
    logical = [logical_kv(kp, vp, bt, b, L0 + T) for b, L0 in enumerate(prompts)]
    for t in range(T):
        lens = torch.tensor([L0 + t + 1 for L0 in prompts], dtype=torch.int32, device="cuda")
        kv = K.PagedKV(kp, vp, bt, lens, P, cap)
        prev = (f64(slots).astype(np.int64), f64(cum), cnt.cpu().numpy().copy())
        out = torch.empty((B, Hq, d), device="cuda")
        K.h2o_step(kv, qs[t].contiguous(), Hq, scale, slots, cum, cnt, 4, 16, 10000, out, budgets=budgets)
        torch.cuda.synchronize()
        s_h, c_h, n_h, o_h = slots.cpu().numpy(), f64(cum), cnt.cpu().numpy(), f64(out)
        for b, L0 in enumerate(prompts):
            Kl, Vl = logical[b]
            for c in range(Hkv):
                # one KV head at a time: its own budget
                sub = (prev[0][:, c:c + 1], prev[1][:, c:c + 1], prev[2][:, c:c + 1])
                _check_step(f64(qs[t, b, c * G:(c + 1) * G]), Kl[c:c + 1], Vl[c:c + 1], L0 + t + 1, sub, b,
                            o_h[b, c * G:(c + 1) * G], None, s_h[:, c:c + 1], c_h[:, c:c + 1], n_h[:, c:c + 1], G,
                            scale, 4, 16, int(budgets[b, c]))
        assert int(cnt[1, 1]) == 20 and int(cnt[0, 0]) == 10000


def test_h2o_lists_seeded_by_the_snapkv_vote():
    """Prefill-vote seeding: the SnapKV vote of the prompt's last 32 queries
    (group sum, pool 7) picks the top-480 prefix positions per KV head; with
    the window they form each list, seeded with their votes (window keys 0).
    Then 4 decode steps of per-step eviction with budget 512 (sinks 4,
    window 64), each checked against the oracle on the GPU's state."""
    K = _K()
    L, W, k, steps = 8192, 32, 480, 4
    cfg = synth.long_context_128k(num_seqs=2, seq_len=L, sparse_steps=steps, device="cuda")
    kvt = cfg["kv"]
    B, Hq, Hkv = 2, 32, 8
    kv0 = K.PagedKV(kvt.k_pages, None, kvt.block_table, kvt.seq_lens, 16, L)
    votes = torch.zeros((B, Hkv, L), device="cuda")
    K.snapkv_vote(kv0, cfg["q_win"], Hq, W, 7, cfg["scale"], K.REDUCE_SUM, votes)
    rows = votes.view(B * Hkv, L)
    keep = torch.empty((B * Hkv, k), dtype=torch.int32, device="cuda")
    kc = torch.empty((B * Hkv,), dtype=torch.int32, device="cuda")
    K.select_keep(rows, torch.full((B * Hkv,), L - W, dtype=torch.int32, device="cuda"), L - W, 0, 0, None, k,
                  keep, kc)
    torch.cuda.synchronize()
    stride = k + W + 8
    slots = torch.zeros((B, Hkv, stride), dtype=torch.int32)
    cum = torch.zeros((B, Hkv, stride))
    vh = votes.cpu()
    for b in range(B):
        for c in range(Hkv):
            lst = torch.cat([keep[b * Hkv + c, :k].cpu(), torch.arange(L - W, L, dtype=torch.int32)])
            slots[b, c, :k + W] = lst
            cum[b, c, :k] = vh[b, c, lst[:k].long()]
    cnt = torch.full((B, Hkv), k + W, dtype=torch.int32)
    slots, cum, cnt = slots.cuda(), cum.cuda(), cnt.cuda()
    logical = [logical_kv(kvt.k_pages, kvt.v_pages, kvt.block_table, b, L + steps) for b in range(B)]
    budget = k + W
    for t in range(steps):
        lens = torch.full((B,), L + t + 1, dtype=torch.int32, device="cuda")
        kv = K.PagedKV(kvt.k_pages, kvt.v_pages, kvt.block_table, lens, 16, L + steps)
        prev = (f64(slots).astype(np.int64), f64(cum), cnt.cpu().numpy().copy())
        out = torch.empty((B, Hq, 128), device="cuda")
        q = cfg["q_dec"][t].contiguous()
        K.h2o_step(kv, q, Hq, cfg["scale"], slots, cum, cnt, 4, 64, budget, out)
        torch.cuda.synchronize()
        s_h, c_h, n_h, o_h = slots.cpu().numpy(), f64(cum), cnt.cpu().numpy(), f64(out)
        for b in range(B):
            Kl, Vl = logical[b]
            _check_step(f64(q[b]), Kl, Vl, L + t + 1, prev, b, o_h[b], None, s_h, c_h, n_h, Hq // Hkv,
                        cfg["scale"], 4, 64, budget)
        assert (cnt == budget).all()
