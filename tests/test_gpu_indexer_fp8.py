"""GPU parity of kvsel_indexer_scores_fp8 against the float64 oracle: the
FP8 E4M3 codes widened by the oracle's own decoder, dot products in float64;
scores within 1e-4 of their error scale sum_d |q_d k_d| (the score tolerance;
the matrix cores' FP8 dot products do not round like a chain of fp32 adds:
about 2e-5 of that scale was seen); the top-2048 chosen on the GPU scores
equal the oracle's selection on those scores."""
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


def _fp8(shape, g, scale):
    return (synth.normal(shape, g) * scale).to(torch.float8_e4m3fn)


@pytest.mark.parametrize("d,G,Hkv,P,lengths,scale", [(64, 32, 1, 16, [5000, 77, 1], 1.0),
                                                      (128, 4, 2, 32, [3000, 1024], 0.125),
                                                      (64, 8, 2, 64, [1500], 0.5)])
def test_indexer_fp8_against_oracle(d, G, Hkv, P, lengths, scale):
    K = _K()
    note(f"fp8 indexer d={d} G={G} Hkv={Hkv} P={P} L={lengths}")
    g = synth.generator(700 + d + G)
    B, Hq, cap = len(lengths), Hkv * G, max(lengths)
    bt, n_pages = synth.shuffled_block_table(B, cap, P, g)
    kp = _fp8((n_pages, Hkv, P, d), g, 2.0)
    q = _fp8((B, Hq, d), g, 2.0)
    kv = K.PagedKV(kp.cuda(), None, bt.cuda(), torch.tensor(lengths, dtype=torch.int32).cuda(), P, cap)
    scores = torch.full((B, Hq, cap + 3), -7.0, device="cuda")
    K.indexer_scores_fp8(kv, q.cuda(), Hq, scale, scores)
    torch.cuda.synchronize()
    kbits = kp.view(torch.uint8).numpy()
    qv = O.fp8_e4m3_bits_to_f64(q.view(torch.uint8).numpy())
    for b, L in enumerate(lengths):
        Kl = O.gather_paged(O.fp8_e4m3_bits_to_f64(kbits), bt[b].numpy(), L)      # [H_kv][L][d]
        for h in range(Hq):
            want = scale * O.indexer_scores(qv[b, h][None, :], Kl[h // G])[0]
            err_scale = scale * (np.abs(Kl[h // G]) @ np.abs(qv[b, h]))
            got = scores[b, h, :L].cpu().double().numpy()
            assert np.all(np.abs(got - want) <= 1e-4 * np.maximum(err_scale, 1e-30))
        assert (scores[b, :, L:] == -7.0).all()


def test_indexer_fp8_top2048_flow():
    """FP8 indexer scores -> top-2048 per query head on 2 x 20000 keys: the
    GPU keep sets equal the oracle's selection on the GPU's scores."""
    K = _K()
    g = synth.generator(777)
    B, Hq, d, P, L = 2, 32, 64, 16, 20000
    bt, n_pages = synth.shuffled_block_table(B, L, P, g)
    kp = _fp8((n_pages, 1, P, d), g, 1.0)
    q = _fp8((B, Hq, d), g, 1.0)
    lens = torch.full((B,), L, dtype=torch.int32)
    kv = K.PagedKV(kp.cuda(), None, bt.cuda(), lens.cuda(), P, L)
    scores = torch.empty((B, Hq, L), device="cuda")
    K.indexer_scores_fp8(kv, q.cuda(), Hq, 1.0, scores)
    rows = scores.view(B * Hq, L)
    keep = torch.empty((B * Hq, 2048), dtype=torch.int32, device="cuda")
    kc = torch.empty((B * Hq,), dtype=torch.int32, device="cuda")
    K.select_keep(rows, torch.full((B * Hq,), L, dtype=torch.int32, device="cuda"), L, 0, 0, None, 2048, keep, kc)
    torch.cuda.synchronize()
    sc = rows.cpu().double().numpy()
    for r in range(0, B * Hq, 7):
        want = O.select_keep(sc[r], L, 0, 0, 2048)
        assert keep[r, :int(kc[r])].cpu().numpy().tolist() == want.tolist()
