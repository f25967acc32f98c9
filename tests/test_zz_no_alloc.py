"""kvsel_decode_attn_scores_noalloc (the entry point for callers that cannot
allocate: its scratch is the library's static device array) gives what the
workspace entry point kvsel_decode_attn_scores gives on the same inputs, on
two calls in a row, the second with a smaller input.  Bars as for decode
parity: out within 2e-3 relative L2, lse / probabilities / cum within 1e-4
relative.  Called through the C ABI (the binding only marshals)."""
import math

import numpy as np
import pytest
import torch

import synth
from tests.parity_util import f64, max_rel, note, rel_l2

pytestmark = pytest.mark.gpu


def _inputs(seed, dtype, B, Hkv, G, d, P, lengths):
    g = synth.generator(seed)
    cap = max(lengths)
    bt, n_pages = synth.shuffled_block_table(B, cap, P, g, extra_pages=2)
    kp = synth.normal((n_pages, Hkv, P, d), g, dtype).cuda()
    vp = synth.normal((n_pages, Hkv, P, d), g, dtype).cuda()
    q = synth.normal((B, Hkv * G, d), g, dtype).cuda()
    lens = torch.tensor(lengths, dtype=torch.int32).cuda()
    return kp, vp, bt.cuda(), lens, q, cap


CASES = [
    # seed, dtype, B, Hkv, G, d, P, lengths, with probs
    (61, torch.bfloat16, 4, 4, 8, 128, 64, [16384, 9000, 1, 12345], True),   # first call, larger
    (62, torch.bfloat16, 2, 2, 4, 128, 16, [1500, 333], False),              # second call, smaller (cum only)
]


def _run(K, case, noalloc):
    seed, dtype, B, Hkv, G, d, P, lengths, with_probs = case
    kp, vp, bt, lens, q, cap = _inputs(seed, dtype, B, Hkv, G, d, P, lengths)
    kv = K.PagedKV(kp, vp, bt, lens, P, cap)
    Hq = Hkv * G
    out = torch.full((B, Hq, d), float("nan"), device="cuda")
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    probs = torch.full((B, Hq, cap), -5.0, device="cuda") if with_probs else None
    g = synth.generator(seed + 1000)
    cum = torch.rand((B, Hkv, cap), generator=g).cuda()
    args = (kv, q, Hq, 1 / math.sqrt(d), out, lse, probs, K.EMIT_PROBS, cum, 0.5)
    if noalloc:
        K.decode_attn_scores_noalloc(*args)
    else:
        K.decode_attn_scores(*args)
    torch.cuda.synchronize()
    return dict(out=out, lse=lse, probs=probs, cum=cum, lengths=lengths)


def test_noalloc_matches_workspace_entry_point():
    import attention_score_guided_amd as K
    for case in CASES:
        note(f"noalloc decode case seed {case[0]} lengths {case[7]}")
        a = _run(K, case, noalloc=True)
        b = _run(K, case, noalloc=False)
        assert rel_l2(f64(a["out"]), f64(b["out"])) < 2e-3
        la, lb = f64(a["lse"]), f64(b["lse"])
        assert (abs(la - lb) <= 1e-4 * np.maximum(1.0, abs(lb))).all()
        for i, L in enumerate(a["lengths"]):
            assert max_rel(f64(a["cum"][i, :, :L]), f64(b["cum"][i, :, :L])) < 1e-4
            assert torch.equal(a["cum"][i, :, L:], b["cum"][i, :, L:])     # untouched past L
            if a["probs"] is not None:
                assert max_rel(f64(a["probs"][i, :, :L]), f64(b["probs"][i, :, :L])) < 1e-4
                assert (a["probs"][i, :, L:] == -5.0).all()
