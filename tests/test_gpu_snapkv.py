"""GPU parity of kvsel_snapkv_vote against the float64 oracle: votes within
1e-4 relative; keep sets chosen on the GPU's votes equal the oracle's
selection on those votes bit for bit."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.parity_util import f64, logical_kv, max_rel, note

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _K():
    import attention_score_guided_amd as K
    return K


CASES = [
    # seed, d, G, Hkv, P, lengths, W, pool, group_sum
    (61, 128, 4, 2, 16, [1500, 700], 32, 7, True),
    (62, 128, 4, 2, 16, [1500, 700], 32, 7, False),
    (63, 64, 2, 2, 64, [999], 7, 3, True),
    (64, 128, 1, 3, 32, [300, 257], 1, 1, True),
    (65, 128, 8, 1, 16, [2100], 40, 7, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}-d{c[1]}-G{c[2]}-W{c[6]}-k{c[7]}-{'sum' if c[8] else 'none'}")
def test_vote_against_oracle(case):
    seed, d, G, Hkv, P, lengths, W, pool, gsum = case
    note(f"snapkv case {case}")
    K = _K()
    g = synth.generator(seed)
    B, Hq = len(lengths), Hkv * G
    bt, n_pages = synth.shuffled_block_table(B, max(lengths), P, g, extra_pages=1)
    kp = synth.normal((n_pages, Hkv, P, d), g, torch.bfloat16).cuda()
    qw = synth.normal((B, Hq, W, d), g, torch.bfloat16).cuda()
    lens = torch.tensor(lengths, dtype=torch.int32).cuda()
    kv = K.PagedKV(kp, None, bt.cuda(), lens, P, max(lengths))
    H = Hkv if gsum else Hq
    stride = max(lengths) + 3
    votes = torch.full((B, H, stride), -9.0, device="cuda")
    K.snapkv_vote(kv, qw, Hq, W, pool, 1 / math.sqrt(d), K.REDUCE_SUM if gsum else K.REDUCE_NONE, votes)
    torch.cuda.synchronize()
    for b, L in enumerate(lengths):
        Kl, _ = logical_kv(kp, None, bt, b, L)
        want = O.snapkv_vote(f64(qw[b]), Kl, 1 / math.sqrt(d), pool, group_sum=gsum)
        got = f64(votes[b, :, :L - W])
        assert max_rel(got, want) < TOL
        assert (votes[b, :, L - W:] == -9.0).all()


def test_vote_long_context_keep_set():
    """Planted long-context data at L = 8192 (4 sequences, 32/8 heads): the
    vote with window 32 and pool 7, then the top-512 per KV head plus the
    window.  Keep sets on the GPU's votes equal the oracle's selection on
    them; the votes match the oracle's; the planted regions dominate."""
    K = _K()
    L, W, k = 8192, 32, 512
    cfg = synth.long_context_128k(seq_len=L, sparse_steps=1, device="cuda")
    kvt = cfg["kv"]
    B, Hq, Hkv = 4, 32, 8
    kv = K.PagedKV(kvt.k_pages, None, kvt.block_table, kvt.seq_lens, 16, L)
    votes = torch.zeros((B, Hkv, L), device="cuda")
    K.snapkv_vote(kv, cfg["q_win"], Hq, W, 7, cfg["scale"], K.REDUCE_SUM, votes)
    rows = votes.view(B * Hkv, L)
    lens = torch.full((B * Hkv,), L - W, dtype=torch.int32, device="cuda")
    keep = torch.empty((B * Hkv, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B * Hkv,), dtype=torch.int32, device="cuda")
    K.select_keep(rows, lens, L - W, 0, 0, None, k, keep, cnt)
    torch.cuda.synchronize()
    gv, kp = f64(votes), keep.cpu().numpy().reshape(B, Hkv, k)
    for b in range(B):
        Kl, _ = logical_kv(kvt.k_pages, None, kvt.block_table, b, L)
        want = O.snapkv_vote(f64(cfg["q_win"][b]), Kl, cfg["scale"], 7, group_sum=True)
        assert max_rel(gv[b, :, :L - W], want) < TOL
        hot = set(range(4))
        for c in cfg["centres"][b]:
            hot |= set(range(c - 255, c + 256))
        for c in range(Hkv):
            want_keep = O.snapkv_keep(gv[b, c, :L - W].astype(np.float32).astype(np.float64), L, W, k)
            got_keep = np.concatenate([kp[b, c], np.arange(L - W, L)])
            np.testing.assert_array_equal(got_keep, want_keep)
            assert np.isin(kp[b, c], list(hot)).mean() > 0.5
