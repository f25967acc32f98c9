"""GPU parity of kvsel_sparse_attn (and the indexer -> top-k -> sparse flow)
against the float64 oracle: outputs within 2e-3 relative L2, listed
probabilities within 1e-4 relative; keep sets chosen on the GPU's own scores
equal the oracle's selection on those same scores bit for bit."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.parity_util import f64, logical_kv, max_rel, note, rel_l2

pytestmark = pytest.mark.gpu
OUT_TOL, SCORE_TOL = 2e-3, 1e-4


def _K():
    import attention_score_guided_amd as K
    return K


def _case(seed, dtype, d, G, Hkv, P, lengths):
    g = synth.generator(seed)
    B = len(lengths)
    bt, n_pages = synth.shuffled_block_table(B, max(lengths), P, g, extra_pages=2)
    kp = synth.normal((n_pages, Hkv, P, d), g, dtype).cuda()
    vp = synth.normal((n_pages, Hkv, P, d), g, dtype).cuda()
    q = synth.normal((B, Hkv * G, d), g, dtype).cuda()
    lens = torch.tensor(lengths, dtype=torch.int32).cuda()
    return kp, vp, bt.cuda(), lens, q


CASES = [
    # seed, dtype, d, G, Hkv, P, lengths, shared, full
    (41, torch.bfloat16, 128, 4, 2, 16, [3000, 700], False, True),
    (42, torch.bfloat16, 128, 4, 2, 16, [3000, 700], True, False),
    (43, torch.bfloat16, 64, 8, 1, 64, [5000], True, False),
    (44, torch.float32, 128, 2, 2, 32, [1000, 999, 4], False, False),
    (45, torch.float32, 64, 1, 3, 16, [600], False, True),
    (46, torch.bfloat16, 128, 8, 2, 16, [9000, 2500], False, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}-d{c[2]}-G{c[3]}-{'shared' if c[7] else 'perhead'}")
def test_sparse_against_oracle(case):
    seed, dtype, d, G, Hkv, P, lengths, shared, full = case
    note(f"sparse case {case}")
    K = _K()
    kp, vp, bt, lens, q = _case(seed, dtype, d, G, Hkv, P, lengths)
    B, Hq = len(lengths), Hkv * G
    idx_heads = Hkv if shared else Hq
    rng = np.random.default_rng(seed)
    stride = max(lengths) + 7
    idx = np.full((B, idx_heads, stride), -1, dtype=np.int32)
    cnt = np.zeros((B, idx_heads), dtype=np.int32)
    for b, L in enumerate(lengths):
        for s in range(idx_heads):
            if full:
                sel = rng.permutation(L)
            else:
                k = int(rng.integers(0, min(L, 2100) + 1)) if s % 3 else min(L, 2048)
                sel = rng.choice(L, size=k, replace=False)
            c = len(sel)
            if not full and c > 3:
                sel = sel.copy()
                sel[rng.integers(0, c, size=3)] = -1         # ignored entries
            idx[b, s, :c] = sel
            cnt[b, s] = c
    max_count = int(cnt.max())
    kv = K.PagedKV(kp, vp, bt, lens, P, max(lengths))
    out = torch.full((B, Hq, d), float("nan"), device="cuda")
    probs = torch.full((B, Hq, stride), -3.0, device="cuda")
    K.sparse_attn(kv, q, Hq, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), max_count,
                  1 / math.sqrt(d), out, probs)
    torch.cuda.synchronize()
    for b, L in enumerate(lengths):
        Kl, Vl = logical_kv(kp, vp, bt, b, L)
        sets = [idx[b, (h // G) if shared else h, :cnt[b, (h // G) if shared else h]] for h in range(Hq)]
        want_out, want_p = O.sparse_attention(f64(q[b]), Kl, Vl, sets, 1 / math.sqrt(d))
        for h in range(Hq):
            c = len(sets[h])
            if (sets[h] >= 0).any():
                assert rel_l2(f64(out[b, h]), want_out[h]) < OUT_TOL
            else:
                assert (out[b, h] == 0).all()
            got_p = f64(probs[b, h, :c])
            nz = want_p[h] > 0
            assert max_rel(got_p[nz], want_p[h][nz]) < SCORE_TOL
            assert (got_p[~nz] == 0).all()
            assert (probs[b, h, c:] == -3.0).all()
        if full:
            dense = O.decode_attention(f64(q[b]), Kl, Vl, 1 / math.sqrt(d))
            assert rel_l2(f64(out[b]), dense["out"]) < OUT_TOL


def test_sparse_empty_sets():
    K = _K()
    kp, vp, bt, lens, q = _case(47, torch.bfloat16, 128, 4, 1, 16, [100])
    idx = torch.full((1, 4, 8), -1, dtype=torch.int32).cuda()
    cnt = torch.tensor([[0, 8, 3, 0]], dtype=torch.int32).cuda()
    out = torch.full((1, 4, 128), float("nan"), device="cuda")
    kv = K.PagedKV(kp, vp, bt, lens, 16, 100)
    K.sparse_attn(kv, q, 4, idx, cnt, 8, 0.1, out)
    torch.cuda.synchronize()
    assert (out == 0).all()


def test_indexer_topk_sparse_flow_long_context():
    """Reduced 128K case (L = 16384): the one-head d=64 indexer scores every
    position (decode in logits mode), each query head keeps its top 2048, and
    sparse attention runs over them.  The GPU's keep sets equal the oracle's
    selection on the GPU's own indexer scores; the indexer scores match the
    oracle's; the sparse outputs match the oracle on the chosen sets."""
    K = _K()
    L, W = 16384, 32
    cfg = synth.long_context_128k(seq_len=L, sparse_steps=1, device="cuda")
    kvt, kit = cfg["kv"], cfg["kv_index"]
    B, Hq, Hkv = 4, 32, 8
    lens = kvt.seq_lens.clone() + 1                      # the first sparse decode step
    kvi = K.PagedKV(kit.k_pages, None, kit.block_table, lens, 16, L + 1)
    qi = cfg["qi_dec"][0].contiguous()
    scores = torch.zeros((B, Hq, L + 1), device="cuda")
    K.decode_attn_scores(kvi, qi, Hq, 1.0, None, None, scores, K.EMIT_LOGITS)
    rows = scores.view(B * Hq, L + 1)
    row_lens = torch.full((B * Hq,), L + 1, dtype=torch.int32, device="cuda")
    keep = torch.empty((B * Hq, 2048), dtype=torch.int32, device="cuda")
    kcnt = torch.empty((B * Hq,), dtype=torch.int32, device="cuda")
    K.select_keep(rows, row_lens, L + 1, 0, 0, None, 2048, keep, kcnt)
    kv = K.PagedKV(kvt.k_pages, kvt.v_pages, kvt.block_table, lens, 16, L + 1)
    q = cfg["q_dec"][0].contiguous()
    out = torch.empty((B, Hq, 128), device="cuda")
    K.sparse_attn(kv, q, Hq, keep.view(B, Hq, 2048), kcnt.view(B, Hq), 2048, cfg["scale"], out)
    torch.cuda.synchronize()
    sc = f64(scores)
    kp = keep.cpu().numpy().reshape(B, Hq, 2048)
    for b in range(B):
        KI, _ = logical_kv(kit.k_pages, None, kit.block_table, b, L + 1)
        want_scores = O.indexer_scores(f64(qi[b]), KI[0])
        assert np.abs(sc[b] - want_scores).max() / np.abs(want_scores).max() < 1e-5
        Kl, Vl = logical_kv(kvt.k_pages, kvt.v_pages, kvt.block_table, b, L + 1)
        sets = []
        for h in range(Hq):
            want_keep = O.select_keep(sc[b, h].astype(np.float32).astype(np.float64), L + 1, 0, 0, 2048)
            np.testing.assert_array_equal(kp[b, h], want_keep)
            sets.append(kp[b, h])
        want_out, _ = O.sparse_attention(f64(q[b]), Kl, Vl, sets, cfg["scale"])
        assert rel_l2(f64(out[b]), want_out) < OUT_TOL
        # the planted hot regions and sinks attract the indexer's top-k
        hot = set()
        for c in cfg["centres"][b]:
            hot |= set(range(c - 255, c + 256))
        frac = np.mean([np.isin(kp[b, h], list(hot | set(range(4)))).mean() for h in range(Hq)])
        assert frac > 0.5


def test_sparse_counts_above_max_count_are_clamped():
    """A count above max_count (a caller error) reads as max_count: only the
    first max_count listed entries take part, every access stays inside the
    index rows, the probability rows and the workspace sized for max_count.
    Compared with the oracle on the clamped sets; probability entries past
    max_count stay untouched."""
    K = _K()
    d, G, Hkv, P, L = 128, 4, 2, 16, 3000
    kp, vp, bt, lens, q = _case(48, torch.bfloat16, d, G, Hkv, P, [L])
    Hq, max_count, stride = Hkv * G, 300, 700
    rng = np.random.default_rng(48)
    idx = np.stack([rng.choice(L, size=stride, replace=False) for _ in range(Hq)]).astype(np.int32)[None]
    cnt = np.array([[stride, max_count + 1, max_count, 17, 513, 299, 300, 301]], dtype=np.int32)
    kv = K.PagedKV(kp, vp, bt, lens, P, L)
    out = torch.full((1, Hq, d), float("nan"), device="cuda")
    probs = torch.full((1, Hq, stride), -3.0, device="cuda")
    K.sparse_attn(kv, q, Hq, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), max_count,
                  1 / math.sqrt(d), out, probs)
    torch.cuda.synchronize()
    Kl, Vl = logical_kv(kp, vp, bt, 0, L)
    used = np.minimum(cnt[0], max_count)
    sets = [idx[0, h, :used[h]] for h in range(Hq)]
    want_out, want_p = O.sparse_attention(f64(q[0]), Kl, Vl, sets, 1 / math.sqrt(d))
    for h in range(Hq):
        assert rel_l2(f64(out[0, h]), want_out[h]) < OUT_TOL
        assert max_rel(f64(probs[0, h, :used[h]]), want_p[h]) < SCORE_TOL
        assert (probs[0, h, used[h]:] == -3.0).all()
