"""GPU parity of kvsel_select_keep against the oracle: keep sets are
bit-exact (the GPU selects on the same fp32 scores the oracle reads)."""
import numpy as np
import pytest
import torch

import oracle as O
from tests.parity_util import note

pytestmark = pytest.mark.gpu


def _K():
    import attention_score_guided_amd as K
    return K


def _run_rows(scores, lengths, sinks, window, budgets, max_budget, per_row_budget=True):
    K = _K()
    rows, stride = scores.shape
    max_len = int(max(lengths))
    out_stride = max(1, min(max_len, max(max_budget, sinks + window)))
    sc = torch.from_numpy(scores.astype(np.float32)).cuda()
    lens = torch.tensor(lengths, dtype=torch.int32).cuda()
    bud = torch.tensor(budgets, dtype=torch.int32).cuda() if per_row_budget else None
    idx = torch.full((rows, out_stride), -5, dtype=torch.int32).cuda()
    cnt = torch.full((rows,), -1, dtype=torch.int32).cuda()
    K.select_keep(sc, lens, max_len, sinks, window, bud, max_budget, idx, cnt)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy()


def _check_rows(scores, lengths, sinks, window, budgets, idx, cnt):
    for r, n in enumerate(lengths):
        want = O.select_keep(scores[r].astype(np.float32).astype(np.float64), n, sinks, window, budgets[r])
        got = idx[r, :cnt[r]]
        assert cnt[r] == len(want), (r, cnt[r], len(want))
        np.testing.assert_array_equal(got, want)
        assert (idx[r, cnt[r]:] == -5).all(), "slots past the count must be untouched"


@pytest.mark.parametrize("seed", range(6))
def test_rows_random_with_ties(seed):
    rng = np.random.default_rng(100 + seed)
    rows = 40
    lengths = [int(x) for x in rng.integers(1, 3000, size=rows)]
    lengths[0], lengths[1], lengths[2] = 1, 2, 3000
    stride = 3001
    scores = rng.integers(0, 50 if seed % 2 else 5, size=(rows, stride)).astype(np.float32)
    if seed == 3:
        scores[scores == 0] = -0.0
        scores[:, ::7] = -np.inf
    sinks, window = [(4, 64), (0, 0), (4, 0), (0, 512), (16, 16), (3000, 0)][seed]
    budgets = [int(rng.integers(0, n + 5)) for n in lengths]
    max_budget = max(budgets)
    note(f"select rows seed={seed} sinks={sinks} window={window}")
    idx, cnt = _run_rows(scores, lengths, sinks, window, budgets, max_budget)
    _check_rows(scores, lengths, sinks, window, budgets, idx, cnt)


def test_rows_shared_budget_and_policies():
    rng = np.random.default_rng(7)
    n, budget = 300, 256
    scores = rng.random((3, n)).astype(np.float32)
    # H2O-style, StreamingLLM (sinks 4 + window 252) and recent-only
    for sinks, window in [(4, 64), (4, budget - 4), (0, budget)]:
        idx, cnt = _run_rows(scores, [n] * 3, sinks, window, [budget] * 3, budget, per_row_budget=False)
        _check_rows(scores, [n] * 3, sinks, window, [budget] * 3, idx, cnt)
    idx, cnt = _run_rows(scores, [n] * 3, 4, budget - 4, [budget] * 3, budget, per_row_budget=False)
    assert idx[0, :cnt[0]].tolist() == list(range(4)) + list(range(n - 252, n))


def test_rows_large_row_top4096():
    """One 131040-key row per KV head, top-4096, nothing forced (the SnapKV
    vote selection shape)."""
    rng = np.random.default_rng(8)
    rows, n = 4, 131040
    scores = rng.random((rows, n)).astype(np.float32)
    scores[1, 1000:2000] = 0.5          # a plateau of ties
    idx, cnt = _run_rows(scores, [n] * rows, 0, 0, [4096] * rows, 4096)
    _check_rows(scores, [n] * rows, 0, 0, [4096] * rows, idx, cnt)


def test_rows_llama3_8b_keep_shape():
    """Per (sequence, KV head) keep budget floor(0.2 L_b) with sinks 4 and
    window 512 over ragged rows of 8K-33K keys."""
    rng = np.random.default_rng(9)
    lens_b = [int(x) for x in rng.integers(8448, 33024, size=16)]
    lengths = [L for L in lens_b for _ in range(8)]
    stride = max(lengths)
    scores = (rng.random((128, stride)) ** 8).astype(np.float32)
    budgets = [int(0.2 * L) for L in lengths]
    idx, cnt = _run_rows(scores, lengths, 4, 512, budgets, max(budgets))
    _check_rows(scores, lengths, 4, 512, budgets, idx, cnt)


GLOBAL_SHAPES = {
    # id: (lengths, global budget); None = drawn from the seed
    "70b_blocks": ([512] * 8, 1024),                               # the 70B block-selection shape
    "shared_rationals": ([4, 8, 16, 12, 6, 24, 3, 48], 31),         # equal keys across rows: row order decides
    "shared_rationals_k0": ([4, 8, 16, 12], 0),
    "all_items": ([7, 1, 300, 64], 372),
    "all_but_one": ([7, 1, 300, 64], 371),
    "single_items": ([1] * 40, 17),
    "many_rows": ([int(x) for x in np.random.default_rng(5).integers(1, 65, size=300)], 4000),
    "past_lds_rows": ([2] * 5000, 3333),                            # more rows than the one-launch search holds
    "random_1": None, "random_2": None, "random_3": None, "random_4": None, "random_5": None,
}


@pytest.mark.parametrize("shape", list(GLOBAL_SHAPES))
def test_global_percentile(shape):
    K = _K()
    seed = list(GLOBAL_SHAPES).index(shape)
    rng = np.random.default_rng(200 + seed)
    if GLOBAL_SHAPES[shape] is not None:
        lengths, gb = GLOBAL_SHAPES[shape]
        rows = len(lengths)
    else:
        rows = int(rng.integers(1, 12))
        lengths = [int(x) for x in rng.integers(1, 700, size=rows)]
        gb = int(rng.integers(0, sum(lengths) + 3))
    max_len = max(lengths)
    scores = rng.integers(0, 6 if seed > 1 else 10**6, size=(rows, max_len)).astype(np.float32)
    sc = torch.from_numpy(scores).cuda()
    lens = torch.tensor(lengths, dtype=torch.int32).cuda()
    idx = torch.full((rows, max_len), -5, dtype=torch.int32).cuda()
    cnt = torch.zeros((rows,), dtype=torch.int32).cuda()
    K.select_keep(sc, lens, max_len, 0, 0, None, 0, idx, cnt, mode=K.SELECT_GLOBAL_PERCENTILE,
                  global_budget=gb)
    torch.cuda.synchronize()
    want = O.global_percentile_select([scores[r].astype(np.float64) for r in range(rows)], lengths, gb)
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for r in range(rows):
        np.testing.assert_array_equal(idx[r, :cnt[r]], want[r])
    assert cnt.sum() == min(gb, sum(lengths))


@pytest.mark.parametrize("seed", range(4))
def test_rows_long_rows_split_over_workgroups(seed):
    """Rows of up to 70K positions (few rows, long rows) with budgets of at
    most 1/8 of a row run the selection split over many workgroups per row;
    keep sets must equal the oracle's,
    including heavy ties across segment boundaries, forced sinks and
    windows, per-row budgets, and a workspace that starts out as junk."""
    K = _K()
    rng = np.random.default_rng(900 + seed)
    rows = 24
    lengths = [int(x) for x in rng.integers(1, 70000, size=rows)]
    lengths[:5] = [1, 16384, 4096 * 7, 69999, 4097]
    lengths[5] = 65536
    stride = 70001
    if seed % 2:
        scores = rng.integers(0, 7, size=(rows, stride)).astype(np.float32)     # heavy ties
    else:
        scores = rng.standard_normal((rows, stride)).astype(np.float32)
        scores[:, 5000:9000] = 1.5                                                # a tied plateau
    sinks, window = [(4, 512), (0, 0), (16, 0), (0, 2048)][seed]
    if seed == 1:
        budgets = [2048] * rows
    elif seed == 3:
        budgets = [int(rng.integers(0, n + 5)) for n in lengths]     # large budgets: per-row kernel
    else:
        budgets = [int(rng.integers(0, min(n + 5, 8000))) for n in lengths]
    max_budget = max(budgets)
    note(f"select long rows seed={seed} sinks={sinks} window={window}")
    max_len = int(max(lengths))
    out_stride = max(1, min(max_len, max(max_budget, sinks + window)))
    sc = torch.from_numpy(scores).cuda()
    lens = torch.tensor(lengths, dtype=torch.int32).cuda()
    bud = None if seed == 1 else torch.tensor(budgets, dtype=torch.int32).cuda()
    nbytes = K.select_workspace_bytes(rows, max_len, K.SELECT_ROWS)
    assert nbytes > 0
    ws = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda")
    for rep in range(2):          # the second call reuses the workspace as the first left it
        idx = torch.full((rows, out_stride), -5, dtype=torch.int32).cuda()
        cnt = torch.full((rows,), -1, dtype=torch.int32).cuda()
        K.select_keep(sc, lens, max_len, sinks, window, bud, max_budget, idx, cnt, workspace=ws)
        torch.cuda.synchronize()
        _check_rows(scores, lengths, sinks, window, budgets, idx.cpu().numpy(), cnt.cpu().numpy())


@pytest.mark.parametrize("case", ["gaussian", "quantised", "fine_ties", "plateau_at_cut", "clustered",
                                  "many_candidates", "dense_segment", "sampled_lines_hot", "sampled_lines_cold",
                                  "cut_far_above_bound"])
def test_rows_long_rows_compaction(case):
    """Long rows with a small keep fraction (the indexer and vote shape): a
    sample of the row bounds the cut from below, the positions at or above
    the bound are compacted per segment and the selection finishes on them.
    Cases cover ties at the threshold (quantised scores: coarsely, so the
    cut's 16-bit bin holds more keys than are ranked directly, or finely, so
    a few dozen keys with repeated values are; or 700 keys equal to the
    cut, more than are ranked directly, with few others stored), kept positions
    clustered in a few segments, a segment whose every position passes,
    more positions at the threshold than the final stage holds, and samples
    that misjudge the row (the sample reads one 16-position line in every
    16): the largest scores only on the sampled lines, so fewer than k
    positions pass the bound, or only off them, so far too many pass (the
    per-row selection takes over in both), or a few thousand scores far
    above the rest only off them, so that the stored positions fit but the
    cut lies far above the bound (the final stage's digits restart from the
    whole key); every result must equal the oracle's."""
    K = _K()
    rng = np.random.default_rng({"gaussian": 11, "quantised": 12, "fine_ties": 19, "plateau_at_cut": 20, "clustered": 13,
                                 "many_candidates": 14, "dense_segment": 15,
                                 "sampled_lines_hot": 16, "sampled_lines_cold": 17,
                                 "cut_far_above_bound": 18}[case])
    rows, n = 6, 131072
    lengths = [n, n - 1, 65536, 100003, 70001, n]
    scores = rng.standard_normal((rows, n)).astype(np.float32)
    budgets = [2048, 2048, 1500, 4096, 777, 2048]
    sinks, window = (4, 512) if case in ("gaussian", "clustered") else (0, 0)
    if case == "quantised":
        scores = np.round(scores * 64.0).astype(np.float32) / 64.0        # heavy ties at tau
    if case == "fine_ties":
        scores = np.round(scores * 2048.0).astype(np.float32) / 2048.0    # ~40 keys per bin at the cut, repeated values
    if case == "plateau_at_cut":
        for r in range(rows):                     # 700 keys equal to the (k - 200)-th largest
            v = np.sort(scores[r, :lengths[r]])[::-1][budgets[r] - 200]
            scores[r, rng.choice(lengths[r], size=700, replace=False)] = v
    if case == "clustered":
        for r in range(rows):                                            # top keys in a few segments
            for c in rng.integers(2000, lengths[r] - 2000, size=3):
                scores[r, c - 300:c + 300] += 4.0
    if case == "many_candidates":
        # ~12% of positions share the threshold's first digit, spread evenly:
        # under the slot cap per segment, but more than the final stage holds
        sel = rng.random((rows, n)) < 0.12
        scores[sel] = (1.0 + 0.18 * rng.random(int(sel.sum()))).astype(np.float32)
        scores[~sel] = np.minimum(scores[~sel], 0.9)
    if case == "dense_segment":
        scores[:, 8192:8192 + 4096] = 3.0 + rng.random((rows, 4096)).astype(np.float32)  # one full segment passes
    on_sampled = (np.arange(n) % 256) < 16
    if case == "sampled_lines_hot":
        scores[:, on_sampled] += 5.0
    if case == "sampled_lines_cold":
        hot = np.zeros(n, dtype=bool)
        for c in rng.integers(0, n // 4096 - 1, size=10):
            hot[c * 4096:(c + 1) * 4096] = True
        scores[:, hot & ~on_sampled] += 5.0
    if case == "cut_far_above_bound":
        off = np.flatnonzero(~on_sampled)
        for r in range(rows):
            scores[r, rng.choice(off[off < lengths[r]], size=3000, replace=False)] += 50.0
    note(f"select compaction case={case}")
    max_budget = max(budgets)
    out_stride = max(max_budget, sinks + window)
    sc = torch.from_numpy(scores).cuda()
    lens = torch.tensor(lengths, dtype=torch.int32).cuda()
    bud = torch.tensor(budgets, dtype=torch.int32).cuda()
    nbytes = K.select_workspace_bytes(rows, n, K.SELECT_ROWS)
    ws = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda")
    for rep in range(2):
        idx = torch.full((rows, out_stride), -5, dtype=torch.int32).cuda()
        cnt = torch.full((rows,), -1, dtype=torch.int32).cuda()
        K.select_keep(sc, lens, n, sinks, window, bud, max_budget, idx, cnt, workspace=ws)
        torch.cuda.synchronize()
        _check_rows(scores, lengths, sinks, window, budgets, idx.cpu().numpy(), cnt.cpu().numpy())
