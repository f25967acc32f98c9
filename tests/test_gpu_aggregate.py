"""GPU parity of kvsel_accumulate and kvsel_block_aggregate against the
float64 oracle (scores within 1e-4 relative)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.parity_util import f64, max_rel, note

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _K():
    import attention_score_guided_amd as K
    return K


@pytest.mark.parametrize("G,Hkv,lengths,decay", [(4, 2, [1, 1000, 4097], 1.0), (8, 1, [333], 0.7),
                                                  (1, 3, [64, 65], 0.0)])
def test_accumulate_standalone(G, Hkv, lengths, decay):
    K = _K()
    g = synth.generator(31)
    B, Hq, stride = len(lengths), G * Hkv, max(lengths) + 3
    probs = torch.rand((B, Hq, stride), generator=g).cuda()
    cum0 = torch.rand((B, Hkv, stride), generator=g).cuda()
    cum = cum0.clone()
    lens = torch.tensor(lengths, dtype=torch.int32).cuda()
    K.accumulate(probs, lens, Hkv, max(lengths), cum, decay)
    torch.cuda.synchronize()
    for b, L in enumerate(lengths):
        want = O.accumulate(f64(cum0[b, :, :L]), f64(probs[b, :, :L]), decay)
        assert max_rel(f64(cum[b, :, :L]), want) < TOL
        assert torch.equal(cum[b, :, L:], cum0[b, :, L:])


@pytest.mark.parametrize("bs,lengths,H", [(16, [1, 15, 16, 17, 528], 2), (64, [32768, 1000], 8),
                                          (7, [100, 49], 3), (256, [1025, 256], 1), (4, [9], 2),
                                          (1, [512, 300, 1], 640), (1, [70], 3)])
@pytest.mark.parametrize("head_sum", [False, True])
def test_block_aggregate(bs, lengths, H, head_sum):
    note(f"block_aggregate bs={bs} L={lengths} H={H} head_sum={head_sum}")
    K = _K()
    g = synth.generator(32)
    B, stride = len(lengths), max(lengths) + 4
    sc = torch.rand((B, H, stride), generator=g).cuda()
    n_blk = -(-max(lengths) // bs)
    shape = (B, n_blk + 2) if head_sum else (B, H, n_blk + 2)
    base_max = torch.rand(shape, generator=g).cuda()
    base_mean = torch.rand(shape, generator=g).cuda()
    lens = torch.tensor(lengths, dtype=torch.int32).cuda()
    red = K.REDUCE_SUM if head_sum else K.REDUCE_NONE
    for acc in (False, True):
        mx, mean = base_max.clone(), base_mean.clone()
        K.block_aggregate(sc, lens, max(lengths), bs, red, acc, mx, mean)
        torch.cuda.synchronize()
        for b, L in enumerate(lengths):
            wm, wa = O.block_aggregate(f64(sc[b]), L, bs)
            nb = wm.shape[1]
            if head_sum:
                wm, wa = wm.sum(0), wa.sum(0)
                gm, ga, bm, ba = f64(mx[b, :nb]), f64(mean[b, :nb]), f64(base_max[b, :nb]), f64(base_mean[b, :nb])
                assert torch.equal(mx[b, nb:], base_max[b, nb:])
            else:
                gm, ga, bm, ba = f64(mx[b, :, :nb]), f64(mean[b, :, :nb]), f64(base_max[b, :, :nb]), f64(base_mean[b, :, :nb])
                assert torch.equal(mx[b, :, nb:], base_max[b, :, nb:])
            if acc:
                wm, wa = wm + bm, wa + ba
            assert max_rel(gm, wm) < TOL and max_rel(ga, wa) < TOL
