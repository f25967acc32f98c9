"""GPU parity of kvsel_union_keep (the KV head keeps the union of its query
heads' picks, SnapKV under GQA) against the oracle: bit-exact, and the
SnapKV per-head flow (votes per query head, top-k per head, union)."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.parity_util import note

pytestmark = pytest.mark.gpu


def _K():
    import attention_score_guided_amd as K
    return K


@pytest.mark.parametrize("max_len,G,Hkv,stride", [(1000, 4, 2, 64), (131072, 4, 2, 4096), (70000, 8, 1, 9000),
                                                  (33, 1, 3, 40)])
def test_union_random_sets(max_len, G, Hkv, stride):
    K = _K()
    note(f"union max_len={max_len} G={G} Hkv={Hkv}")
    rng = np.random.default_rng(max_len + G)
    B, Hq = 2, G * Hkv
    idx = np.full((B, Hq, stride), -1, dtype=np.int32)
    cnt = np.zeros((B, Hq), dtype=np.int32)
    for b in range(B):
        for h in range(Hq):
            n = int(rng.integers(0, stride + 1))
            vals = rng.choice(max_len, size=min(n, max_len), replace=False) if h % 3 else \
                rng.integers(0, max_len // 2 + 1, size=n)            # repeats inside a list, overlaps across
            vals = np.sort(vals)[:n].astype(np.int32)
            if len(vals) > 2:
                vals[1] = -1                                           # ignored entry
            idx[b, h, :len(vals)] = vals
            cnt[b, h] = len(vals)
    out_stride = min(max_len, G * stride) + 5
    out = torch.full((B, Hkv, out_stride), -9, dtype=torch.int32, device="cuda")
    oc = torch.empty((B, Hkv), dtype=torch.int32, device="cuda")
    K.union_keep(torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), Hkv, max_len, out, oc)
    torch.cuda.synchronize()
    for b in range(B):
        for c in range(Hkv):
            want = O.union_keep([idx[b, h, :cnt[b, h]] for h in range(c * G, (c + 1) * G)])
            n = int(oc[b, c])
            assert out[b, c, :n].cpu().numpy().tolist() == want.tolist()
            assert (out[b, c, n:] == -9).all()


def test_snapkv_per_head_picks_and_union():
    """Votes per query head (no group reduce), the top-k per query head, then
    the union per KV head, on the long-context synthetic cache (2 x 8192
    keys, 32 / 8 heads, window 32, pool 7, top-256)."""
    K = _K()
    L, W, k = 8192, 32, 256
    cfg = synth.long_context_128k(num_seqs=2, seq_len=L, sparse_steps=1, device="cuda")
    kvt = cfg["kv"]
    Hq, Hkv = 32, 8
    kv = K.PagedKV(kvt.k_pages, None, kvt.block_table, kvt.seq_lens, 16, L)
    votes = torch.zeros((2, Hq, L), device="cuda")
    K.snapkv_vote(kv, cfg["q_win"], Hq, W, 7, cfg["scale"], K.REDUCE_NONE, votes)
    rows = votes.view(2 * Hq, L)
    lens = torch.full((2 * Hq,), L - W, dtype=torch.int32, device="cuda")
    keep = torch.empty((2 * Hq, k), dtype=torch.int32, device="cuda")
    kc = torch.empty((2 * Hq,), dtype=torch.int32, device="cuda")
    K.select_keep(rows, lens, L - W, 0, 0, None, k, keep, kc)
    out = torch.empty((2, Hkv, 4 * k), dtype=torch.int32, device="cuda")
    oc = torch.empty((2, Hkv), dtype=torch.int32, device="cuda")
    K.union_keep(keep.view(2, Hq, k), kc.view(2, Hq), Hkv, L, out, oc)
    torch.cuda.synchronize()
    v = votes.cpu().double().numpy()
    for b in range(2):
        for c in range(Hkv):
            picks = [O.select_keep(v[b, h], L - W, 0, 0, k) for h in range(c * 4, (c + 1) * 4)]
            want = O.union_keep(picks)
            n = int(oc[b, c])
            assert out[b, c, :n].cpu().numpy().tolist() == want.tolist()
            assert k <= n <= 4 * k
