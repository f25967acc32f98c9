"""GPU parity of the score-aggregation variants (kvsel_accumulate_ex,
kvsel_block_aggregate_ex, kvsel_select_threshold) against the float64
oracle: scores within 1e-5 relative (block top-p% means: tree sums),
fractions, flags and index sets exact except decisions on values within
1e-6 of the threshold."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.parity_util import f64, max_rel, note

pytestmark = pytest.mark.gpu


def _K():
    import attention_score_guided_amd as K
    return K


def _probs(g, B, Hq, stride, lengths):
    p = torch.rand((B, Hq, stride), generator=g)
    for b, L in enumerate(lengths):
        p[b, :, :L] /= p[b, :, :L].sum(dim=1, keepdim=True)
        p[b, :, L:] = 0.5          # past the row: must be ignored
    return p


@pytest.mark.parametrize("G", [1, 4])
def test_accumulate_max_and_window_over_steps(G):
    K = _K()
    g = synth.generator(91 + G)
    Hkv, lengths, steps, W = 2, [700, 33, 1], 7, 3
    B, Hq, stride = len(lengths), Hkv * G, 704
    lens = torch.tensor(lengths, dtype=torch.int32).cuda()
    cum_max = torch.zeros((B, Hkv, stride), device="cuda")
    cum_win = torch.full((B, Hkv, stride), -2.0, device="cuda")
    ring = torch.zeros((W, B, Hkv, stride), device="cuda")
    o_max = [np.zeros((Hkv, L)) for L in lengths]
    hist = [[] for _ in lengths]
    for t in range(steps):
        p = _probs(g, B, Hq, stride, lengths)
        pc = p.cuda()
        K.accumulate_ex(pc, lens, Hkv, max(lengths), cum_max, K.ACC_MAX, decay=0.9)
        K.accumulate_ex(pc, lens, Hkv, max(lengths), cum_win, K.ACC_WINDOW_MEAN, window=W, step=t, ring=ring)
        torch.cuda.synchronize()
        for b, L in enumerate(lengths):
            pb = p[b, :, :L].double().numpy()
            o_max[b] = O.accumulate_max(o_max[b], pb, 0.9)
            o_win = O.accumulate_window(hist[b], pb, Hkv, W)
            assert max_rel(f64(cum_max[b, :, :L]), o_max[b]) < 1e-5
            assert max_rel(f64(cum_win[b, :, :L]), o_win) < 1e-5
            assert (cum_win[b, :, L:] == -2.0).all()


@pytest.mark.parametrize("bs,param", [(16, 0.25), (4, 0.5), (32, 0.1), (64, 0.1), (256, 0.5), (5, 1.0)])
def test_block_variants(bs, param):
    K = _K()
    note(f"block variants bs={bs} p={param}")
    g = synth.generator(95 + bs)
    lengths, H = [1000, 77, 3], 3
    B, stride = len(lengths), 1003
    sc = torch.rand((B, H, stride), generator=g)
    sc[0, 0, :64] = 0.5                                   # ties inside blocks
    lens = torch.tensor(lengths, dtype=torch.int32).cuda()
    n_blk = -(-max(lengths) // bs)
    scd = sc.cuda()
    outs = {}
    for mode, prm in [(K.BLOCK_TOP_P_MEAN, param), (K.BLOCK_FRAC_ABOVE, 0.6), (K.BLOCK_ALL_COLD, 0.97)]:
        out = torch.full((B, H, n_blk + 2), -1.0, device="cuda")
        K.block_aggregate_ex(scd, lens, max(lengths), bs, mode, prm, out)
        outs[mode] = out
    torch.cuda.synchronize()
    for b, L in enumerate(lengths):
        nb = -(-L // bs)
        for h in range(H):
            row = sc[b, h].double().numpy()
            assert max_rel(f64(outs[K.BLOCK_TOP_P_MEAN][b, h, :nb]), O.block_top_p_mean(row, L, bs, param)) < 1e-5
            assert np.array_equal(f64(outs[K.BLOCK_FRAC_ABOVE][b, h, :nb]),
                                  O.block_fraction_above(row.astype(np.float32), L, bs, np.float32(0.6)).astype(np.float32))
            assert np.array_equal(f64(outs[K.BLOCK_ALL_COLD][b, h, :nb]),
                                  O.block_all_cold(row.astype(np.float32), L, bs, np.float32(0.97)))
            for m in outs:
                assert (outs[m][b, h, nb:] == -1.0).all()


def test_select_threshold_rows():
    K = _K()
    g = synth.generator(99)
    lengths = [5000, 1, 256, 257, 0 + 3]
    rows, stride = len(lengths), 5004
    sc = torch.rand((rows, stride), generator=g)
    sc[2] = 0.7                                           # every position exactly at the threshold
    lens = torch.tensor(lengths, dtype=torch.int32).cuda()
    idx = torch.full((rows, stride), -5, dtype=torch.int32, device="cuda")
    cnt = torch.empty((rows,), dtype=torch.int32, device="cuda")
    K.select_threshold(sc.cuda(), lens, max(lengths), 0.7, idx, cnt)
    torch.cuda.synchronize()
    for r, L in enumerate(lengths):
        want = O.select_threshold(sc[r].numpy(), L, np.float32(0.7))
        n = int(cnt[r])
        assert idx[r, :n].cpu().numpy().tolist() == want.tolist()
        assert (idx[r, n:] == -5).all()


@pytest.mark.parametrize("bs,decay,weighted", [(16, 0.9, True), (64, 1.0, False), (1, 0.5, True), (5, 0.7, True)])
def test_block_update_over_steps(bs, decay, weighted):
    """kvsel_block_update over 6 steps of fresh ascending lists (ragged counts,
    an empty row, a row of padding only, -1 entries inside lists, a block
    whose entries straddle a padding run past the workgroup's staged range,
    a block size that is not a power of two): stamps exact, scores within
    1e-5 relative of the oracle, records past the last block untouched."""
    K = _K()
    note(f"block_update bs={bs} decay={decay} weighted={weighted}")
    rng = np.random.default_rng(300 + bs)
    L = 3000
    nb = -(-L // bs)
    counts_base = [0, 1, 2048, 5, 777, 40, 354]
    # row 6: entry 250 opens a block, 100 padding entries, then two more
    # entries of the same block (at 351, 352: past the 320 staged entries)
    straddle = np.array([-1] * 250 + [320] + [-1] * 100 + [321, 322] + [2999], dtype=np.int32)
    rows, stride = len(counts_base), 2048 + 16
    sc_o = [np.zeros(nb) for _ in range(rows)]
    st_o = [np.zeros(nb, dtype=np.int64) for _ in range(rows)]
    meta = K.block_meta(rows, nb + 3)
    score, stamp = K.block_meta_views(meta)
    for step in range(1, 7):
        idx = np.full((rows, stride), -1, dtype=np.int32)
        vals = np.full((rows, stride), 7.0, dtype=np.float32)
        cnt = np.zeros(rows, dtype=np.int32)
        for r, c in enumerate(counts_base):
            sel = np.sort(rng.choice(L, size=c, replace=False)).astype(np.int32)
            if r == 5:
                lst = np.full(c, -1, dtype=np.int32)              # padding only
            elif r == 6:
                lst = straddle
            else:
                lst = np.insert(sel, rng.integers(0, c + 1, size=min(c, 9)), -1) if c else sel
            idx[r, :len(lst)] = lst
            vals[r, :len(lst)] = rng.random(len(lst))
            cnt[r] = len(lst)
        ti, tc = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
        tv = torch.from_numpy(vals).cuda() if weighted else None
        K.block_update(ti, tc, bs, step, meta, tv, decay)
        for r in range(rows):
            lst = idx[r, :cnt[r]]
            sc_o[r], st_o[r] = O.block_update(sc_o[r], st_o[r], lst, vals[r, :cnt[r]] if weighted else None, bs,
                                              step, decay)
    torch.cuda.synchronize()
    for r in range(rows):
        assert stamp[r, :nb].cpu().numpy().tolist() == st_o[r].tolist()
        assert max_rel(f64(score[r, :nb]), sc_o[r]) < 1e-5
        assert score[r, nb:].abs().sum().item() == 0 and stamp[r, nb:].abs().sum().item() == 0
