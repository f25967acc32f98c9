"""The seeded generators are deterministic and plant what they claim."""
import hashlib
import math

import numpy as np
import torch

import synth


def _digest(*ts):
    h = hashlib.sha256()
    for t in ts:
        h.update(t.contiguous().view(torch.uint8).numpy().tobytes() if t.dtype != torch.int32
                 else t.numpy().tobytes())
    return h.hexdigest()


def test_tiny_case_deterministic_and_sink_bias():
    a, b = synth.tiny_case(), synth.tiny_case()
    assert _digest(a["kv"].k_pages, a["kv"].v_pages, a["q_steps"], a["kv"].block_table) == \
        _digest(b["kv"].k_pages, b["kv"].v_pages, b["q_steps"], b["kv"].block_table)
    kv = a["kv"]
    bt = kv.block_table[0].long()
    K = torch.stack([kv.k_pages[bt[j // 16], 0, j % 16] for j in range(528)]).double()
    q = a["q_steps"][:, 0].double()                        # [steps][Hq][d]
    logits = (q @ K.T) * a["scale"]                        # [steps][Hq][528]
    # the planted direction: sink keys minus a generic key's share along the query
    u = q[0, 0] / q[0, 0].norm()
    # every query carries sqrt(d) along u0, so sinks lead non-sink keys by ~4 on average
    gap = logits[..., :4].mean() - logits[..., 4:].mean()
    assert 3.5 < float(gap) < 4.5
    assert u.shape[0] == 64


def test_shuffled_block_table_is_a_partial_permutation():
    g = synth.generator(7)
    bt, n = synth.shuffled_block_table(5, 100, 16, g, extra_pages=3)
    assert bt.shape == (5, 7) and n == 38
    flat = bt.flatten().tolist()
    assert len(set(flat)) == len(flat) and max(flat) < n and min(flat) >= 0


def test_llama3_8b_layer_small_deterministic():
    a = synth.llama3_8b_layer(num_seqs=2, min_len=64, max_len=200, steps=4)
    b = synth.llama3_8b_layer(num_seqs=2, min_len=64, max_len=200, steps=4)
    assert torch.equal(a["kv"].k_pages.view(torch.int16), b["kv"].k_pages.view(torch.int16))
    assert torch.equal(a["q_steps"].view(torch.int16), b["q_steps"].view(torch.int16))
    assert a["kv"].seq_lens.min() >= 64 and a["kv"].seq_lens.max() <= 200
    t = a["temperature"]
    assert float(t.min()) >= 0.5 and float(t.max()) <= 2.0
