"""Pins of the float64 oracle to facts that do not come from the oracle itself.

Each test checks one oracle function against a closed form, an invariant, a
library routine, a brute-force enumeration or a value printed on the pages,
chosen so that a dropped term, a wrong sign, a wrong GQA index or a transposed
operand fails at least one of them.  CPU only.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.ndimage
import scipy.special

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


# ----------------------------------------------------------------- O1 decode
def test_decode_single_key_closed_form():
    d = 8
    q = np.zeros((1, d)); q[0, 0] = 2.0
    K = np.zeros((1, 1, d)); K[0, 0, 0] = 3.0
    V = rng.normal(size=(1, 1, d))
    r = O.decode_attention(q, K, V, 0.5)
    assert r["probs"][0, 0] == 1.0
    np.testing.assert_array_equal(r["out"][0], V[0, 0])
    assert r["logits"][0, 0] == 3.0          # 0.5 * 2 * 3
    assert r["lse"][0] == 3.0                # ln(e^3)


@pytest.mark.parametrize("a", [-3.0, 0.0, 0.7, 5.0])
def test_decode_two_keys_is_logistic(a):
    d, scale = 4, 0.25
    q = np.zeros((1, d)); q[0, 0] = a
    K = np.zeros((1, 2, d)); K[0, 0, 0] = 1.0          # s0 = scale*a, s1 = 0
    V = np.zeros((1, 2, d)); V[0, 0, 1] = 1.0; V[0, 1, 2] = 1.0
    r = O.decode_attention(q, K, V, scale)
    p0 = 1.0 / (1.0 + math.exp(-scale * a))
    assert abs(r["probs"][0, 0] - p0) < 1e-15
    assert abs(r["probs"][0, 1] - (1 - p0)) < 1e-15
    assert abs(r["out"][0, 1] - p0) < 1e-15 and abs(r["out"][0, 2] - (1 - p0)) < 1e-15
    assert abs(r["lse"][0] - math.log(math.exp(scale * a) + 1.0)) < 1e-14


def test_decode_equal_keys_uniform():
    Hq, Hkv, L, d = 4, 2, 37, 16
    q = rng.normal(size=(Hq, d))
    K = np.repeat(rng.normal(size=(Hkv, 1, d)), L, axis=1)
    V = rng.normal(size=(Hkv, L, d))
    r = O.decode_attention(q, K, V, 0.3)
    np.testing.assert_allclose(r["probs"], 1.0 / L, rtol=1e-14)
    for h in range(Hq):
        np.testing.assert_allclose(r["out"][h], V[h // 2].mean(axis=0), rtol=1e-12, atol=1e-14)


def test_decode_matches_scipy_softmax_and_logsumexp():
    Hq, Hkv, L, d = 8, 2, 300, 64
    q = rng.normal(size=(Hq, d)); K = rng.normal(size=(Hkv, L, d)); V = rng.normal(size=(Hkv, L, d))
    scale = 1 / math.sqrt(d)
    r = O.decode_attention(q, K, V, scale)
    G = Hq // Hkv
    for h in range(Hq):
        s = np.array([scale * sum(q[h, t] * K[h // G, j, t] for t in range(d)) for j in range(L)])
        np.testing.assert_allclose(r["logits"][h], s, rtol=1e-12, atol=1e-12)
        p = scipy.special.softmax(s)
        np.testing.assert_allclose(r["probs"][h], p, rtol=1e-12, atol=1e-15)
        assert abs(r["lse"][h] - scipy.special.logsumexp(s)) < 1e-12
        np.testing.assert_allclose(r["out"][h], np.einsum("j,jd->d", p, V[h // G]), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(r["probs"].sum(axis=1), 1.0, rtol=1e-13)


def test_decode_gqa_head_mapping_repeat_interleave():
    # KV head c has constant value c+1: query head h must read head h // G.
    Hq, Hkv, L, d = 12, 3, 20, 8
    q = rng.normal(size=(Hq, d)); K = rng.normal(size=(Hkv, L, d))
    V = np.stack([np.full((L, d), c + 1.0) for c in range(Hkv)])
    r = O.decode_attention(q, K, V, 0.5)
    for h in range(Hq):
        np.testing.assert_allclose(r["out"][h], h // 4 + 1.0, rtol=1e-13)


def test_decode_stable_for_huge_logits_and_permutation_invariant():
    d = 4
    q = np.array([[100.0, 0, 0, 0]])
    K = np.zeros((1, 3, d)); K[0, 0, 0] = 100.0; K[0, 1, 0] = -100.0
    r = O.decode_attention(q, K, None, 1.0)
    assert np.isfinite(r["probs"]).all() and abs(r["probs"][0, 0] - 1.0) < 1e-15
    assert r["out"] is None
    # permuting keys permutes probs and leaves out unchanged
    Hq, L = 2, 50
    q = rng.normal(size=(Hq, d)); K = rng.normal(size=(1, L, d)); V = rng.normal(size=(1, L, d))
    perm = rng.permutation(L)
    a = O.decode_attention(q, K, V, 0.9); b = O.decode_attention(q, K[:, perm], V[:, perm], 0.9)
    np.testing.assert_allclose(b["probs"], a["probs"][:, perm], rtol=1e-13)
    np.testing.assert_allclose(b["out"], a["out"], rtol=1e-12, atol=1e-14)


def test_gather_paged_inverts_a_scatter():
    Hkv, P, d, L = 3, 16, 8, 70
    logical = rng.normal(size=(Hkv, L, d))
    n_pages = 9
    bt = rng.permutation(n_pages)[:5]
    pages = rng.normal(size=(n_pages, Hkv, P, d))
    for j in range(L):                       # test-side scatter, slot by slot
        pages[bt[j // P], :, j % P, :] = logical[:, j, :]
    np.testing.assert_array_equal(O.gather_paged(pages, bt, L), logical)


def test_bf16_widening_exact():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0x3E00, 0x0001], dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, math.inf, 0.125, 2.0 ** -133]
    got = O.bf16_bits_to_f64(bits)
    for g, w in zip(got, want):
        assert g == w and math.copysign(1, g) == math.copysign(1, w)


# -------------------------------------------------------------- O2 accumulate
def test_accumulate_group_mapping_one_hot():
    Hq, Hkv, L = 8, 2, 8
    probs = np.eye(Hq, L)                   # head h puts all mass on key h
    cum = O.accumulate(np.zeros((Hkv, L)), probs)
    for c in range(Hkv):
        for j in range(L):
            assert cum[c, j] == (1.0 if j // 4 == c else 0.0)


def test_accumulate_sums_to_steps_times_query_heads():
    Hq, Hkv, L, d, steps = 6, 3, 40, 16, 7
    cum = np.zeros((Hkv, L))
    for _ in range(steps):
        r = O.decode_attention(rng.normal(size=(Hq, d)), rng.normal(size=(Hkv, L, d)), None, 0.25)
        cum = O.accumulate(cum, r["probs"])
    assert abs(cum.sum() - steps * Hq) < 1e-11


def test_accumulate_decay_geometric_series():
    Hq, Hkv, L, n, delta = 4, 2, 5, 9, 0.8
    p = rng.random((Hq, L))
    cum = np.zeros((Hkv, L))
    for _ in range(n):
        cum = O.accumulate(cum, p, decay=delta)
    group = p.reshape(Hkv, 2, L).sum(axis=1)
    np.testing.assert_allclose(cum, group * (1 - delta ** n) / (1 - delta), rtol=1e-13)


# ---------------------------------------------------------- O3 block aggregate
def test_block_aggregate_hand_example():
    mx, mean = O.block_aggregate(np.array([[1.0, 2, 3, 4, 5, 99]]), 5, 2)
    np.testing.assert_array_equal(mx, [[2, 4, 5]])
    np.testing.assert_array_equal(mean, [[1.5, 3.5, 5]])


@pytest.mark.parametrize("L,bs", [(1, 16), (16, 16), (17, 16), (100, 7), (528, 16), (255, 64)])
def test_block_aggregate_against_masked_reshape(L, bs):
    H = 3
    x = rng.random((H, L + 5))
    mx, mean = O.block_aggregate(x, L, bs)
    n_blk = -(-L // bs)
    pad = np.full((H, n_blk * bs), np.nan)
    pad[:, :L] = x[:, :L]
    r = pad.reshape(H, n_blk, bs)
    np.testing.assert_array_equal(mx, np.nanmax(r, axis=2))
    np.testing.assert_allclose(mean, np.nanmean(r, axis=2), rtol=1e-14)
    assert (mx >= mean - 1e-15).all()
    counts = np.minimum(bs, L - np.arange(n_blk) * bs)
    assert abs((mean * counts).sum() - x[:, :L].sum()) < 1e-10


# ----------------------------------------------------------------- O4 select
def _brute_keep(sc, n, s, w, budget):
    """Independent definition: a middle item is a heavy hitter iff fewer than
    k middle items beat it (higher score, or equal score and lower index)."""
    if budget >= n:
        return list(range(n))
    forced = [j for j in range(n) if j < s or j >= n - w]
    k = max(0, budget - len(forced))
    mid = [j for j in range(n) if j not in forced]
    keep = set(forced)
    for j in mid:
        beat = sum(1 for i in mid if sc[i] > sc[j] or (sc[i] == sc[j] and i < j))
        if beat < k:
            keep.add(j)
    return sorted(keep)


def test_select_hand_example_h2o():
    sc = np.array([5.0, 1, 9, 2, 8, 3, 7, 4])
    # sinks {0}, window {6,7}, heavy hitters = 2 best of positions 1..5 -> 2, 4
    assert O.select_keep(sc, 8, 1, 2, 5).tolist() == [0, 2, 4, 6, 7]


def test_select_budget_at_least_n_keeps_all():
    sc = rng.random(50)
    for b in (50, 51, 1000):
        assert O.select_keep(sc, 50, 4, 8, b).tolist() == list(range(50))


def test_select_streaming_and_recent_sets_exact():
    n, budget = 300, 256
    sc = rng.random(n)
    got = O.select_keep(sc, n, 4, budget - 4, budget)
    assert got.tolist() == list(range(4)) + list(range(n - 252, n))
    assert O.streaming_keep(n, budget).tolist() == got.tolist()
    got = O.select_keep(sc, n, 0, budget, budget)
    assert got.tolist() == list(range(n - budget, n)) == O.recent_keep(n, budget).tolist()
    assert O.streaming_keep(200, 256).tolist() == list(range(200))


def test_select_against_brute_force_with_ties():
    for trial in range(300):
        n = int(rng.integers(1, 25))
        sc = rng.integers(0, 4, size=n).astype(float)        # many ties
        if trial % 3 == 0:
            sc[sc == 0] = -0.0                                  # -0 equals +0
        s, w = int(rng.integers(0, 5)), int(rng.integers(0, 5))
        budget = int(rng.integers(0, n + 3))
        got = O.select_keep(sc, n, s, w, budget).tolist()
        assert got == _brute_keep(sc, n, s, w, budget), (sc, s, w, budget)
        if budget < n:
            forced = len(set(range(min(s, n))) | set(range(max(n - w, 0), n)))
            assert len(got) == max(budget, forced)


def test_select_neg_inf_is_lowest():
    sc = np.array([-np.inf, 1.0, -np.inf, 0.5])
    assert O.select_keep(sc, 4, 0, 0, 2).tolist() == [1, 3]
    assert O.select_keep(sc, 4, 0, 0, 3).tolist() == [0, 1, 3]


# ------------------------------------------------------- O5 global percentile
def test_percentile_hand_example():
    keys = O.percentile_keys(np.array([0.3, 0.1, 0.3, 0.2]), 4)
    assert keys == [Fraction(4, 4), Fraction(1, 4), Fraction(3, 4), Fraction(2, 4)]


def test_global_percentile_brute_force():
    for _ in range(60):
        R = int(rng.integers(1, 5))
        lens = [int(rng.integers(1, 9)) for _ in range(R)]
        rows = [rng.integers(0, 3, size=n).astype(float) for n in lens]
        K = int(rng.integers(0, sum(lens) + 2))
        got = O.global_percentile_select(rows, lens, K)
        cand = []
        for r, n in enumerate(lens):
            for j in range(n):
                below = sum(1 for i in range(n)
                            if rows[r][i] < rows[r][j] or (rows[r][i] == rows[r][j] and i > j))
                cand.append((Fraction(below + 1, n), r, j))
        want = [[] for _ in lens]
        for key, r, j in cand:
            better = sum(1 for k2, r2, j2 in cand
                         if k2 > key or (k2 == key and (r2, j2) < (r, j)))
            if better < K:
                want[r].append(j)
        assert [g.tolist() for g in got] == [sorted(w) for w in want]


def test_global_percentile_equal_lengths_is_per_row_topk():
    R, n, frac = 8, 512, 0.25
    rows = [rng.random(n) for _ in range(R)]
    got = O.global_percentile_select(rows, [n] * R, int(frac * R * n))
    for r in range(R):
        assert got[r].tolist() == O.select_keep(rows[r], n, 0, 0, int(frac * n)).tolist()


# ---------------------------------------------------------------- O6 SnapKV
@pytest.mark.parametrize("k", [1, 3, 7, 9])
def test_max_pool_matches_scipy(k):
    x = rng.normal(size=57)
    want = scipy.ndimage.maximum_filter1d(x, size=k, mode="constant", cval=-np.inf)
    np.testing.assert_array_equal(O.max_pool_1d(x, k), want)


def test_snapkv_window_one_equals_decode_probs():
    Hq, Hkv, L, d = 4, 2, 64, 16
    K = rng.normal(size=(Hkv, L, d)); q = rng.normal(size=(Hq, 1, d))
    v = O.snapkv_vote(q, K, 0.25, 1, group_sum=False)
    r = O.decode_attention(q[:, 0], K, None, 0.25)
    np.testing.assert_allclose(v, r["probs"][:, :L - 1], rtol=1e-13)


def test_snapkv_two_window_rows_are_causal():
    Hq, Hkv, L, d = 2, 1, 40, 8
    K = rng.normal(size=(Hkv, L, d)); q = rng.normal(size=(Hq, 2, d))
    v = O.snapkv_vote(q, K, 0.5, 1, group_sum=False)
    a = O.decode_attention(q[:, 0], K[:, :L - 1], None, 0.5)["probs"][:, :L - 2]
    b = O.decode_attention(q[:, 1], K, None, 0.5)["probs"][:, :L - 2]
    np.testing.assert_allclose(v, a + b, rtol=1e-13)


def test_snapkv_votes_sum_to_window_when_window_keys_are_cold():
    Hq, Hkv, L, W, d = 4, 2, 80, 8, 16
    q0 = rng.normal(size=d)
    q = np.broadcast_to(q0, (Hq, W, d)).copy()
    K = rng.normal(size=(Hkv, L, d)) * 0.1
    K[:, L - W:] = -40.0 * q0 / np.linalg.norm(q0)        # window keys get ~zero mass
    per_head = O.snapkv_vote(q, K, 1.0, 1, group_sum=False)
    np.testing.assert_allclose(per_head.sum(axis=1), W, rtol=1e-9)
    grouped = O.snapkv_vote(q, K, 1.0, 1, group_sum=True)
    np.testing.assert_allclose(grouped, per_head.reshape(Hkv, 2, -1).sum(axis=1), rtol=1e-13)
    pooled = O.snapkv_vote(q, K, 1.0, 7, group_sum=True)
    np.testing.assert_array_equal(
        pooled, scipy.ndimage.maximum_filter1d(grouped, size=7, axis=1, mode="constant", cval=-np.inf))


def test_snapkv_keep_is_topk_plus_window():
    vote = rng.random(100)
    keep = O.snapkv_keep(vote, 110, 10, 5)
    top5 = np.argsort(-vote, kind="stable")[:5]
    assert keep.tolist() == sorted(top5.tolist()) + list(range(100, 110))


# --------------------------------------------------------------- O7 indexer
def test_indexer_brute_force():
    H, L, dI = 3, 11, 5
    q = rng.normal(size=(H, dI)); K = rng.normal(size=(L, dI))
    s = O.indexer_scores(q, K)
    for h in range(H):
        for j in range(L):
            assert abs(s[h, j] - sum(q[h, t] * K[j, t] for t in range(dI))) < 1e-12


# ---------------------------------------------------------------- O8 sparse
def test_sparse_full_set_equals_dense():
    Hq, Hkv, L, d = 8, 2, 90, 32
    q = rng.normal(size=(Hq, d)); K = rng.normal(size=(Hkv, L, d)); V = rng.normal(size=(Hkv, L, d))
    dense = O.decode_attention(q, K, V, 0.2)
    sets = [rng.permutation(L) for _ in range(Hq)]
    out, probs = O.sparse_attention(q, K, V, sets, 0.2)
    np.testing.assert_allclose(out, dense["out"], rtol=1e-12, atol=1e-14)
    for h in range(Hq):
        np.testing.assert_allclose(probs[h], dense["probs"][h][sets[h]], rtol=1e-12)


def test_sparse_single_key_and_padding():
    Hq, Hkv, L, d = 2, 1, 30, 8
    q = rng.normal(size=(Hq, d)); K = rng.normal(size=(Hkv, L, d)); V = rng.normal(size=(Hkv, L, d))
    out, probs = O.sparse_attention(q, K, V, [[-1, 7, -1], [3]], 0.3)
    np.testing.assert_array_equal(out[0], V[0, 7])
    np.testing.assert_array_equal(out[1], V[0, 3])
    assert probs[0].tolist() == [0.0, 1.0, 0.0]


def test_relative_error_values():
    assert O.relative_error(np.array([1.0, 1.0]), np.array([1.0, 0.0])) == 1.0
    assert O.relative_error(np.array([3.0, 4.0]), np.array([3.0, 4.0])) == 0.0


# ------------------------------------------------- sparse-comparison index sets
def test_window_index_sets_hand():
    assert O.window_index_set(10, 4).tolist() == [7, 8, 9, 10]
    assert O.window_index_set(2, 4).tolist() == [0, 1, 2]
    assert O.sink_window_index_set(20, 8, 4).tolist() == [0, 1, 2, 3, 17, 18, 19, 20]
    assert O.sink_window_index_set(5, 8, 4).tolist() == [0, 1, 2, 3, 4, 5]


def test_quest_picks_the_page_of_a_dominant_key_and_keeps_the_tail():
    L, d, page = 70, 8, 16
    q = rng.normal(size=d)
    K = rng.normal(size=(L, d)) * 0.01
    K[37] = 50 * q                          # page 2 holds the dominant key
    sel = O.quest_page_selection(q, K, 69, 16, page)
    assert sel.tolist() == list(range(32, 48)) + list(range(64, 70))
    sel = O.quest_page_selection(q, K, 40, 16, page)     # causal cut at 40
    assert sel.tolist() == list(range(32, 41))
    # the bound dominates every key's score of the page
    for pg in range(L // page):
        blk = K[pg * page:(pg + 1) * page]
        bound = np.maximum(q * blk.min(0), q * blk.max(0)).sum()
        assert (blk @ q <= bound + 1e-12).all()


def test_quest_summary_is_the_page_min_and_max():
    # hand example: two whole pages of 2 keys, one partial page
    K = np.array([[1.0, -2.0], [3.0, 0.5], [-1.0, 4.0], [-1.0, 4.0], [9.0, 9.0]])
    kmin, kmax = O.quest_page_summary(K, 2)
    assert kmin.tolist() == [[1.0, -2.0], [-1.0, 4.0]]
    assert kmax.tolist() == [[3.0, 0.5], [-1.0, 4.0]]


def test_quest_bound_is_the_box_maximum_by_brute_force():
    # sum_d max(q_d*lo_d, q_d*hi_d) is the maximum of q.x over the box
    # [lo, hi]; a linear function peaks at a corner, so enumerate all 2^d.
    d = 6
    for trial in range(20):
        q = rng.normal(size=d)
        K = rng.normal(size=(32, d))
        kmin, kmax = O.quest_page_summary(K, 16)
        bounds = O.quest_page_bounds(q, kmin, kmax)
        for pg in range(2):
            corners = [np.where([(m >> i) & 1 for i in range(d)], kmax[pg], kmin[pg]) for m in range(1 << d)]
            assert bounds[pg] == pytest.approx(max(c @ q for c in corners), rel=1e-12, abs=1e-12)
            assert (K[pg * 16:(pg + 1) * 16] @ q <= bounds[pg] + 1e-12).all()


def test_quest_bound_sign_cases_and_tightness():
    K = rng.normal(size=(48, 5))
    kmin, kmax = O.quest_page_summary(K, 16)
    qp = np.abs(rng.normal(size=5))
    np.testing.assert_allclose(O.quest_page_bounds(qp, kmin, kmax), kmax @ qp, rtol=1e-13)
    np.testing.assert_allclose(O.quest_page_bounds(-qp, kmin, kmax), kmin @ -qp, rtol=1e-13)
    # a page of identical keys: the bound is the exact score
    Ke = np.repeat(rng.normal(size=(1, 5)), 16, axis=0)
    q = rng.normal(size=5)
    assert O.quest_page_bounds(q, *O.quest_page_summary(Ke, 16))[0] == pytest.approx(Ke[0] @ q, rel=1e-13)


def test_h2o_evict_step_hand_example():
    # one head, d = 1, q = 1, scale 1: logits are the key values themselves.
    # Prompt keys 3, 0, 2 all kept; the new key 1 joins; budget 2, window 1:
    # forced = the new slot, one heavy hitter among positions 0..2 -> position 0.
    K = np.array([[[3.0], [0.0], [2.0], [1.0]]])
    V = np.array([[[10.0], [20.0], [30.0], [40.0]]])
    out, probs, kept, cum = O.h2o_evict_step(np.array([[1.0]]), K, V, [[0, 1, 2]], [np.zeros(3)], 1.0,
                                             0, 1, 2)
    e = np.exp([3.0, 0.0, 2.0, 1.0])
    p = e / e.sum()
    np.testing.assert_allclose(probs[0], p, rtol=1e-15)
    assert out[0, 0] == pytest.approx(p @ [10, 20, 30, 40], rel=1e-14)
    assert kept[0].tolist() == [0, 3]
    np.testing.assert_allclose(cum[0], [p[0], p[3]], rtol=1e-15)


def _h2o_run(T, L0, Hq, Hkv, d, sinks, window, budget, seed=5):
    r = np.random.default_rng(seed)
    K = r.normal(size=(Hkv, L0 + T, d))
    V = r.normal(size=(Hkv, L0 + T, d))
    qs = r.normal(size=(T, Hq, d))
    kept = [np.arange(L0) for _ in range(Hkv)]
    cum = [np.zeros(L0) for _ in range(Hkv)]
    hist = []
    for t in range(T):
        L = L0 + t + 1
        out, probs, kept, cum = O.h2o_evict_step(qs[t], K[:, :L], V[:, :L], kept, cum, 0.3, sinks, window,
                                                 budget)
        hist.append((out, probs, [k.copy() for k in kept], [c.copy() for c in cum]))
    return K, V, qs, hist


def test_h2o_evict_without_eviction_is_full_decode_and_accumulate():
    # budget above every length: no eviction, so each step is full decode
    # attention and the scores are the plain accumulated probabilities
    T, L0, Hq, Hkv, d = 6, 9, 4, 2, 5
    K, V, qs, hist = _h2o_run(T, L0, Hq, Hkv, d, 2, 3, 1000)
    cum = np.zeros((Hkv, L0 + T))
    for t, (out, probs, kept, c) in enumerate(hist):
        L = L0 + t + 1
        r = O.decode_attention(qs[t], K[:, :L], V[:, :L], 0.3)
        np.testing.assert_allclose(out, r["out"], rtol=1e-12, atol=1e-14)
        cum[:, :L] = O.accumulate(cum[:, :L], r["probs"])
        for ci in range(Hkv):
            assert kept[ci].tolist() == list(range(L))
            np.testing.assert_allclose(c[ci], cum[ci, :L], rtol=1e-12)


def test_h2o_evict_with_sinks_and_window_filling_the_budget_is_streaming():
    # sinks + window = budget leaves no heavy hitter: StreamingLLM's list
    T, L0, budget = 12, 20, 10
    _, _, _, hist = _h2o_run(T, L0, 2, 1, 4, 4, budget - 4, budget)
    for t, (_, probs, kept, cum) in enumerate(hist):
        L = L0 + t + 1
        assert kept[0].tolist() == O.streaming_keep(L, budget, 4).tolist()
        assert all(abs(p.sum() - 1) < 1e-12 for p in probs)


def test_h2o_evict_invariants_with_heavy_hitters():
    T, L0, Hq, Hkv, budget = 10, 30, 4, 2, 12
    _, _, _, hist = _h2o_run(T, L0, Hq, Hkv, 6, 2, 3, budget)
    mass = 0.0
    for t, (_, probs, kept, cum) in enumerate(hist):
        L = L0 + t + 1
        for ci in range(Hkv):
            assert len(kept[ci]) == budget
            assert kept[ci][:2].tolist() == [0, 1] and kept[ci][-3:].tolist() == [L - 3, L - 2, L - 1]
            assert (np.diff(kept[ci]) > 0).all()
        # scores only ever gain mass while kept, and lose a slot's when evicted
        assert sum(c.sum() for c in cum) <= (t + 1) * Hq + 1e-9
        assert all(abs(p.sum() - 1) < 1e-12 for p in probs)


def test_accumulate_max_and_window_closed_forms():
    probs = rng.uniform(size=(6, 4, 9))              # 6 steps, 4 query heads, 9 keys
    probs /= probs.sum(axis=2, keepdims=True)
    cum_max = np.zeros((2, 9))
    hist = []
    for t in range(6):
        cum_max = O.accumulate_max(cum_max, probs[t])
        win = O.accumulate_window(hist, probs[t], 2, 3)
        g = probs[:t + 1].reshape(t + 1, 2, 2, 9).sum(axis=2)     # group sums so far
        np.testing.assert_allclose(cum_max, g.max(axis=0), rtol=1e-15)
        np.testing.assert_allclose(win, g[-3:].sum(axis=0) / 3, rtol=1e-14)
    # decay 0 keeps only the current step; window 1 is the current step too
    np.testing.assert_allclose(O.accumulate_max(np.full((2, 9), 5.0), probs[0], 0.0),
                               probs[0].reshape(2, 2, 9).sum(axis=1), rtol=1e-15)


def test_block_variants_limits_and_hand_values():
    sc = np.array([0.1, 0.9, 0.3, 0.3, 0.2, 0.0, 0.7])
    # top-p mean: p -> 0 is the block max, p = 1 the block mean
    mx, mean = O.block_aggregate(sc[None, :], 7, 3)
    np.testing.assert_allclose(O.block_top_p_mean(sc, 7, 3, 1e-9), mx[0], rtol=1e-15)
    np.testing.assert_allclose(O.block_top_p_mean(sc, 7, 3, 1.0), mean[0], rtol=1e-15)
    assert O.block_top_p_mean(sc, 7, 3, 0.5).tolist() == pytest.approx([0.6, 0.25, 0.7])   # top 2 of 3
    assert O.block_fraction_above(sc, 7, 3, 0.3).tolist() == pytest.approx([2 / 3, 1 / 3, 1.0])
    assert O.block_all_cold(sc, 7, 3, 0.3).tolist() == [0.0, 0.0, 0.0]
    assert O.block_all_cold(sc, 7, 3, 0.35).tolist() == [0.0, 1.0, 0.0]
    assert O.select_threshold(sc, 7, 0.3).tolist() == [1, 2, 3, 6]
    assert O.select_threshold(sc, 5, 2.0).tolist() == []


def test_block_update_hand_example_lazy_decay_and_counts():
    # blocks of 4; positions 1, 2 | 5 | 12, 13 with weights; block 2 untouched
    sc, st = O.block_update([1.0, 2.0, 3.0, 4.0], [0, 1, 0, 2], [1, 2, -1, 5, 12, 13],
                            [0.1, 0.2, 9.0, 0.3, 0.4, 0.5], 4, 3, 0.5)
    np.testing.assert_allclose(sc, [1.0 * 0.125 + 0.3, 2.0 * 0.25 + 0.3, 3.0, 4.0 * 0.5 + 0.9])
    assert st.tolist() == [3, 3, 0, 3]
    # lazy ageing = eager ageing of every block at every step, read out at the end
    rng = np.random.default_rng(5)
    nb, bs, d = 6, 8, 0.8
    lazy_s, lazy_t = np.zeros(nb), np.zeros(nb, dtype=np.int64)
    eager = np.zeros(nb)
    for step in range(1, 12):
        lst = np.sort(rng.choice(nb * bs, size=7, replace=False))
        w = rng.random(7)
        lazy_s, lazy_t = O.block_update(lazy_s, lazy_t, lst, w, bs, step, d)
        eager *= d
        np.add.at(eager, lst // bs, w)
    np.testing.assert_allclose(lazy_s * d ** (11 - lazy_t), eager, rtol=1e-12)
    # decay 1, unit weights: the hit count of every block
    lst = np.sort(rng.choice(64, size=20, replace=False))
    sc, _ = O.block_update(np.zeros(8), np.zeros(8, dtype=np.int64), lst, None, 8, 1)
    assert sc.tolist() == np.bincount(lst // 8, minlength=8).astype(float).tolist()


def test_union_keep_hand_example_and_library_union():
    assert O.union_keep([[3, 1, -1], [1, 7], []]).tolist() == [1, 3, 7]
    sets = [rng.integers(-3, 50, size=int(n)) for n in rng.integers(0, 30, size=5)]
    want = np.unique(np.concatenate([s[s >= 0] for s in sets] + [np.array([], dtype=np.int64)]))
    assert O.union_keep(sets).tolist() == want.tolist()


def test_fp8_e4m3_decoding():
    # codes fixed by the format: 1.0, the largest finite 448, the smallest
    # subnormal 2^-9, the smallest normal 2^-6, signed zero, NaN
    v = O.fp8_e4m3_bits_to_f64(np.array([0x38, 0x7E, 0x01, 0x08, 0x00, 0x80, 0xB8, 0x7F, 0xFF]))
    assert v[:7].tolist() == [1.0, 448.0, 2.0 ** -9, 2.0 ** -6, 0.0, 0.0, -1.0]
    assert np.signbit(v[5]) and np.isnan(v[7]) and np.isnan(v[8])
    # every code against torch's float8_e4m3fn widening (a library routine)
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.fp8_e4m3_bits_to_f64(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])


# ------------------------------------------------------------ chunk attention
def test_chunk_causal_attention_rows():
    Hq, Hkv, S, n, d = 4, 2, 10, 5, 8
    qc = rng.normal(size=(Hq, n, d))
    Kc, Vc = rng.normal(size=(Hkv, S, d)), rng.normal(size=(Hkv, S, d))
    Kn, Vn = rng.normal(size=(Hkv, n, d)), rng.normal(size=(Hkv, n, d))
    out, probs = O.chunk_causal_attention(qc, Kc, Vc, Kn, Vn, 0.3)
    assert [p.shape[1] for p in probs] == [S + i + 1 for i in range(n)]
    full = O.decode_attention(qc[:, n - 1], np.concatenate([Kc, Kn], 1), np.concatenate([Vc, Vn], 1), 0.3)
    np.testing.assert_allclose(out[n - 1], full["out"], rtol=1e-13)
    first = O.decode_attention(qc[:, 0], np.concatenate([Kc, Kn[:, :1]], 1),
                               np.concatenate([Vc, Vn[:, :1]], 1), 0.3)
    np.testing.assert_allclose(out[0], first["out"], rtol=1e-13)


# ------------------------------------------------------------ printed values
def test_cost_model_reproduces_printed_values():
    g = json.load(open(os.path.join(GOLDEN, "longctx_cost_model.json")))
    for m in g["models"]:
        cross = O.attention_linear_crossover(m["params"], m["layers"], m["heads"], m["head_dim"])
        assert round(cross / 1000) == m["crossover_k"]
        kv = O.kv_bytes_per_token(m["layers"], m["kv_heads"], m["head_dim"]) * 131072 / 1e9
        assert round(kv, 1) == m["kv_128k_gb"]
        # at the crossover, attention FLOPs per token equal 2*params
        fl = O.attention_flops_per_token(cross, m["layers"], m["heads"], m["head_dim"])
        assert abs(fl - 2 * m["params"]) < 1e-3 * m["params"]


def test_decode_read_estimate_of_offloading_page():
    g = json.load(open(os.path.join(GOLDEN, "offload_decode_read.json")))
    m = g["model"]
    gb = O.kv_bytes_per_token(m["layers"], m["kv_heads"], m["head_dim"], m["bytes_per_elt"]) * g["context"] / 1e9
    assert abs(gb - g["kv_read_gb_approx"]) / g["kv_read_gb_approx"] < 0.1
    ms = gb / g["hbm_tb_per_s"]
    assert abs(ms - g["time_ms_approx"]) / g["time_ms_approx"] < 0.1
