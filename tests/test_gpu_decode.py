"""GPU parity of kvsel_decode_attn_scores (+ fused accumulation) against the
float64 oracle, through the C ABI.

Bars (from the method's accuracy requirements): attention outputs within
2e-3 relative L2 (bf16 in, fp32 accumulation); probabilities, log-sum-exp and
cumulative scores within 1e-4 relative.  Raw logits within 1e-5 relative to
the logit scale.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.parity_util import f64, logical_kv, logical_kv_rows, max_rel, note, rel_l2

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-3
SCORE_TOL = 1e-4


def _K():
    import attention_score_guided_amd as K
    return K


def _random_case(seed, dtype, d, G, Hkv, P, lengths, extra_stride=0, device="cuda"):
    g = synth.generator(seed)
    B = len(lengths)
    cap = max(lengths)
    bt, n_pages = synth.shuffled_block_table(B, cap, P, g, extra_pages=3)
    kp = synth.normal((n_pages, Hkv, P, d), g, dtype)
    vp = synth.normal((n_pages, Hkv, P, d), g, dtype)
    q = synth.normal((B, Hkv * G, d), g, dtype)
    lens = torch.tensor(lengths, dtype=torch.int32)
    return dict(kp=kp.to(device), vp=vp.to(device), bt=bt.to(device), lens=lens.to(device),
                q=q.to(device), Hq=Hkv * G, P=P, max_len=cap, stride=cap + extra_stride,
                scale=1 / math.sqrt(d))


def _oracle(c, b, with_v=True):
    L = int(c["lens"][b])
    K_, V_ = logical_kv(c["kp"], c["vp"] if with_v else None, c["bt"], b, L)
    return O.decode_attention(f64(c["q"][b]), K_, V_, c["scale"])


CASES = [
    # seed, dtype, d, G, Hkv, P, lengths
    (11, torch.bfloat16, 128, 4, 2, 16, [1, 63, 513, 1500]),
    (12, torch.bfloat16, 128, 8, 2, 64, [4096, 700]),
    (13, torch.bfloat16, 64, 2, 4, 32, [65, 1024, 64]),
    (14, torch.float32, 128, 1, 3, 256, [300, 257]),
    (15, torch.float32, 64, 16, 1, 16, [1000, 2]),
    (16, torch.bfloat16, 128, 32, 1, 16, [777]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}-{str(c[1])[6:]}-d{c[2]}-G{c[3]}-P{c[5]}")
def test_decode_all_outputs(case):
    seed, dtype, d, G, Hkv, P, lengths = case
    note(f"decode parity case seed={seed} dtype={dtype} d={d} G={G} Hkv={Hkv} P={P} L={lengths}")
    K = _K()
    c = _random_case(seed, dtype, d, G, Hkv, P, lengths, extra_stride=5)
    B, Hq = len(lengths), c["Hq"]
    kv = K.PagedKV(c["kp"], c["vp"], c["bt"], c["lens"], P, c["max_len"])
    out = torch.full((B, Hq, d), float("nan"), device="cuda")
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    probs = torch.full((B, Hq, c["stride"]), -7.0, device="cuda")
    cum0 = torch.rand((B, Hkv, c["stride"]), device="cuda")
    cum = cum0.clone()
    K.decode_attn_scores(kv, c["q"], Hq, c["scale"], out, lse, probs, K.EMIT_PROBS, cum, 0.5)
    torch.cuda.synchronize()
    for b in range(B):
        L = lengths[b]
        r = _oracle(c, b)
        assert rel_l2(f64(out[b]), r["out"]) < OUT_TOL
        for h in range(Hq):
            assert rel_l2(f64(out[b, h]), r["out"][h]) < OUT_TOL
        assert max_rel(f64(lse[b]), r["lse"]) < SCORE_TOL
        assert max_rel(f64(probs[b, :, :L]), r["probs"]) < SCORE_TOL
        assert (probs[b, :, L:] == -7.0).all(), "probs past L_b must be untouched"
        want = O.accumulate(f64(cum0[b, :, :L]), r["probs"], decay=0.5)
        assert max_rel(f64(cum[b, :, :L]), want) < SCORE_TOL
        assert torch.equal(cum[b, :, L:], cum0[b, :, L:])


@pytest.mark.parametrize("G,extra", [(32, 0), (32, 1), (24, 2), (32, 3)])
def test_decode_logits_mode_without_values(G, extra):
    """Indexer-style call: one KV head, G query heads (24: a partial second
    column tile), d=64, raw logits, no V; row strides that are not 16-byte
    aligned take the staged store path, whose writes stay inside [0, L_b)."""
    K = _K()
    note(f"logits mode G={G} stride extra={extra}")
    c = _random_case(21, torch.bfloat16, 64, G, 1, 16, [3000, 17, 1024], extra_stride=extra)
    kv = K.PagedKV(c["kp"], None, c["bt"], c["lens"], 16, c["max_len"])
    logits = torch.full((3, G, c["stride"]), -7.0, device="cuda")
    K.decode_attn_scores(kv, c["q"], G, 1.0, None, None, logits, K.EMIT_LOGITS)
    torch.cuda.synchronize()
    for b, L in enumerate([3000, 17, 1024]):
        Kl, _ = logical_kv(c["kp"], None, c["bt"], b, L)
        want = O.indexer_scores(f64(c["q"][b]), Kl[0])
        err = np.abs(f64(logits[b, :, :L]) - want).max() / np.abs(want).max()
        assert err < 1e-5
        assert (logits[b, :, L:] == -7.0).all()


def test_decode_cum_without_probs_uses_scratch_and_lse_only():
    K = _K()
    c = _random_case(22, torch.bfloat16, 128, 4, 2, 16, [2500, 900])
    kv = K.PagedKV(c["kp"], None, c["bt"], c["lens"], 16, c["max_len"])
    cum = torch.zeros((2, 2, c["stride"]), device="cuda")
    lse = torch.zeros((2, 8), device="cuda")
    K.decode_attn_scores(kv, c["q"], 8, c["scale"], None, lse, None, K.EMIT_PROBS, cum, 1.0)
    torch.cuda.synchronize()
    for b, L in enumerate([2500, 900]):
        r = _oracle(c, b, with_v=False)
        assert max_rel(f64(lse[b]), r["lse"]) < SCORE_TOL
        want = O.accumulate(np.zeros((2, L)), r["probs"])
        assert max_rel(f64(cum[b, :, :L]), want) < SCORE_TOL
        assert abs(float(cum[b].sum()) - 8.0) < 1e-3


def test_decode_bitwise_deterministic():
    K = _K()
    c = _random_case(23, torch.bfloat16, 128, 8, 2, 16, [5000, 3333])
    kv = K.PagedKV(c["kp"], c["vp"], c["bt"], c["lens"], 16, c["max_len"])
    res = []
    for _ in range(2):
        out = torch.empty((2, 16, 128), device="cuda")
        probs = torch.empty((2, 16, c["stride"]), device="cuda")
        cum = torch.ones((2, 2, c["stride"]), device="cuda")
        K.decode_attn_scores(kv, c["q"], 16, c["scale"], out, None, probs, K.EMIT_PROBS, cum, 1.0)
        torch.cuda.synchronize()
        res.append((out, probs[:, :, :3333], cum[:, :, :3333]))
    for a, b in zip(*res):
        assert torch.equal(a, b)


def test_tiny_case_sixteen_steps_with_h2o_accumulation():
    """Tiny case: 1 sequence, G=4, d=64, fp32, 512-token prompt with planted
    sinks, 16 decode steps each appending a token; cum accumulated on the GPU
    with the fused path, compared step by step with the oracle."""
    K = _K()
    cfg = synth.tiny_case(device="cuda")
    kvt = cfg["kv"]
    steps, prompt, Hq = cfg["steps"], cfg["prompt"], cfg["num_q_heads"]
    cap = prompt + steps
    lens = torch.empty(1, dtype=torch.int32, device="cuda")
    cum = torch.zeros((1, 1, cap), device="cuda")
    cum_ref = np.zeros((1, cap))
    Kall, Vall = logical_kv(kvt.k_pages, kvt.v_pages, kvt.block_table, 0, cap)
    for s in range(steps):
        L = prompt + s + 1
        lens.fill_(L)
        kv = K.PagedKV(kvt.k_pages, kvt.v_pages, kvt.block_table, lens, 16, cap)
        out = torch.empty((1, Hq, 64), device="cuda")
        probs = torch.zeros((1, Hq, cap), device="cuda")
        q = cfg["q_steps"][s].contiguous()
        K.decode_attn_scores(kv, q, Hq, cfg["scale"], out, None, probs, K.EMIT_PROBS, cum, 1.0)
        torch.cuda.synchronize()
        r = O.decode_attention(f64(q[0]), Kall[:, :L], Vall[:, :L], cfg["scale"])
        assert rel_l2(f64(out[0]), r["out"]) < OUT_TOL
        assert max_rel(f64(probs[0, :, :L]), r["probs"]) < SCORE_TOL
        cum_ref[:, :L] = O.accumulate(cum_ref[:, :L], r["probs"])
        assert max_rel(f64(cum[0, :, :L]), cum_ref[:, :L]) < SCORE_TOL
    assert abs(float(cum.sum()) - steps * Hq) < 1e-3
    # the planted sinks dominate the accumulated scores
    assert float(cum[0, 0, :4].min()) > float(cum[0, 0, 4:].max())


def test_llama3_8b_layer_reduced_steps_ragged():
    """Llama-3-8B-shape layer scaled down (B=4, L_b in [1000, 3000]): 8 decode
    steps appending one key per step, fused accumulation, q / T_b."""
    K = _K()
    steps = 8
    cfg = synth.llama3_8b_layer(num_seqs=4, min_len=1000, max_len=3000, steps=steps, device="cuda")
    kvt = cfg["kv"]
    B, Hq, Hkv = 4, 32, 8
    base = kvt.seq_lens.clone()
    cap = int(base.max()) + steps
    cum = torch.zeros((B, Hkv, cap), device="cuda")
    cum_ref = [np.zeros((Hkv, int(base[b]) + steps)) for b in range(B)]
    logical = [logical_kv(kvt.k_pages, kvt.v_pages, kvt.block_table, b, int(base[b]) + steps) for b in range(B)]
    for s in range(steps):
        lens = (base + s + 1).to(torch.int32)
        kv = K.PagedKV(kvt.k_pages, kvt.v_pages, kvt.block_table, lens, 16, cap)
        out = torch.empty((B, Hq, 128), device="cuda")
        q = cfg["q_steps"][s].contiguous()
        K.decode_attn_scores(kv, q, Hq, cfg["scale"], out, None, None, K.EMIT_PROBS, cum, 1.0)
        torch.cuda.synchronize()
        for b in range(B):
            L = int(lens[b])
            Kl, Vl = logical[b]
            r = O.decode_attention(f64(q[b]), Kl[:, :L], Vl[:, :L], cfg["scale"])
            assert rel_l2(f64(out[b]), r["out"]) < OUT_TOL
            cum_ref[b][:, :L] = O.accumulate(cum_ref[b][:, :L], r["probs"])
    for b in range(B):
        L = int(base[b]) + steps
        assert max_rel(f64(cum[b, :, :L]), cum_ref[b][:, :L]) < SCORE_TOL
        assert abs(float(cum[b].sum()) - steps * Hq) < 1e-2


def test_llama70b_layer_full_size_sampled():
    """LLaMA-70B-shape layer at full size (B=8, L=32768, G=8, P=64) in the
    launch configuration the benchmark times (probs emitted, cum fused):
    sampled (sequence, KV head) rows are checked in full against the oracle
    and the probability mass of every sequence against H_q."""
    K = _K()
    cfg = synth.llama70b_layer(0, device="cuda")
    kvt = cfg["kv"]
    B, Hq, Hkv, L = 8, 64, 8, 32768
    kv = K.PagedKV(kvt.k_pages, kvt.v_pages, kvt.block_table, kvt.seq_lens, 64, L)
    out = torch.empty((B, Hq, 128), device="cuda")
    lse = torch.empty((B, Hq), device="cuda")
    probs = torch.empty((B, Hq, L), device="cuda")
    cum = torch.zeros((B, Hkv, L), device="cuda")
    K.decode_attn_scores(kv, cfg["q"], Hq, cfg["scale"], out, lse, probs, K.EMIT_PROBS, cum, 1.0)
    torch.cuda.synchronize()
    sums = cum.double().sum(dim=(1, 2)).cpu().numpy()
    np.testing.assert_allclose(sums, Hq, rtol=1e-4)
    for b, c in [(0, 0), (5, 3), (7, 7)]:
        Kl, Vl = logical_kv_rows(kvt.k_pages, kvt.v_pages, kvt.block_table, b, c, L)
        hs = slice(c * 8, c * 8 + 8)
        r = O.decode_attention(f64(cfg["q"][b, hs]), Kl, Vl, cfg["scale"])
        assert rel_l2(f64(out[b, hs]), r["out"]) < OUT_TOL
        assert max_rel(f64(lse[b, hs]), r["lse"]) < SCORE_TOL
        assert max_rel(f64(probs[b, hs]), r["probs"]) < SCORE_TOL
        assert max_rel(f64(cum[b, c]), r["probs"].sum(axis=0)) < SCORE_TOL


@pytest.mark.parametrize("wait_us", [0, 40], ids=["fallback", "in-kernel"])
def test_decode_normalisation_paths_and_workspace_reuse(wait_us):
    """The bf16 pass normalises in-kernel once all chunks of a (sequence, KV
    head) row have posted their (max, sum); a workgroup that stops waiting
    hands its chunk to the fix-up pass.  A wait bound of 0 forces a mix of both
    (only the last chunk of a row to arrive sees the row complete).  One
    workspace, first filled with junk, serves three calls in a row so stale
    arrival words of earlier calls are exercised."""
    K = _K()
    c = _random_case(31, torch.bfloat16, 128, 8, 2, 16, [5000, 1, 2049, 4096])
    B, Hq, Hkv = 4, 16, 2
    kv = K.PagedKV(c["kp"], c["vp"], c["bt"], c["lens"], 16, c["max_len"])
    nbytes = K.decode_workspace_bytes(kv, Hq, True)
    ws = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda")
    prev = K.set_sync_wait_us(wait_us)
    try:
        cum = torch.zeros((B, Hkv, c["stride"]), device="cuda")
        for it in range(3):
            out = torch.empty((B, Hq, 128), device="cuda")
            probs = torch.full((B, Hq, c["stride"]), -3.0, device="cuda")
            K.decode_attn_scores(kv, c["q"], Hq, c["scale"], out, None, probs, K.EMIT_PROBS, cum, 1.0,
                                 workspace=ws)
            torch.cuda.synchronize()
            for b, L in enumerate([5000, 1, 2049, 4096]):
                r = _oracle(c, b)
                assert rel_l2(f64(out[b]), r["out"]) < OUT_TOL
                assert max_rel(f64(probs[b, :, :L]), r["probs"]) < SCORE_TOL
                assert (probs[b, :, L:] == -3.0).all()
                want = (it + 1) * r["probs"].reshape(Hkv, Hq // Hkv, L).sum(axis=1)
                assert max_rel(f64(cum[b, :, :L]), want) < SCORE_TOL
    finally:
        K.set_sync_wait_us(prev)


def test_decode_cum_only_fallback_uses_scratch():
    """cum without probs on the forced fix-up path: chunk values go through
    the workspace scratch rows."""
    K = _K()
    c = _random_case(32, torch.bfloat16, 64, 4, 3, 32, [3100, 700])
    kv = K.PagedKV(c["kp"], None, c["bt"], c["lens"], 32, c["max_len"])
    prev = K.set_sync_wait_us(0)
    try:
        cum = torch.zeros((2, 3, c["stride"]), device="cuda")
        K.decode_attn_scores(kv, c["q"], 12, c["scale"], None, None, None, K.EMIT_PROBS, cum, 1.0)
        torch.cuda.synchronize()
    finally:
        K.set_sync_wait_us(prev)
    for b, L in enumerate([3100, 700]):
        r = _oracle(c, b, with_v=False)
        want = r["probs"].reshape(3, 4, L).sum(axis=1)
        assert max_rel(f64(cum[b, :, :L]), want) < SCORE_TOL


AGG_CASES = [
    # seed, dtype, d, G, Hkv, P, lengths, block, wait bound in us (None: default)
    (41, torch.bfloat16, 128, 8, 2, 64, [4096, 1500, 64], 64, None),    # fused in the pass
    (42, torch.bfloat16, 128, 4, 3, 16, [2049, 777], 16, None),
    (43, torch.bfloat16, 64, 2, 2, 32, [3000, 100], 256, None),
    (44, torch.bfloat16, 128, 8, 2, 64, [4096, 1500], 64, 0),            # chunks finished by the fix-up
    (45, torch.float32, 128, 4, 2, 16, [1000, 333], 16, None),          # aggregation after the pass
    (46, torch.bfloat16, 128, 4, 2, 16, [2000, 1111], 48, None),         # block size not a power of two
]


@pytest.mark.parametrize("case", AGG_CASES, ids=lambda c: f"s{c[0]}-{str(c[1])[6:]}-G{c[3]}-bs{c[7]}-wait{c[8]}")
def test_decode_with_block_aggregates(case):
    """kvsel_decode_attn_scores_agg: probabilities and cum as the plain call,
    plus the block max / mean of the updated cum per (sequence, KV head),
    written into a strided array (two 'layers' stacked as extra heads)."""
    seed, dtype, d, G, Hkv, P, lengths, bs, wait_us = case
    note(f"decode+agg case {case}")
    K = _K()
    c = _random_case(seed, dtype, d, G, Hkv, P, lengths, extra_stride=3)
    B, Hq = len(lengths), c["Hq"]
    kv = K.PagedKV(c["kp"], c["vp"], c["bt"], c["lens"], P, c["max_len"])
    n_blk = -(-c["max_len"] // bs)
    head_stride = n_blk + 2
    layers = 2
    seq_stride = layers * Hkv * head_stride + 5
    blk_max = torch.full((B * seq_stride,), -9.0, device="cuda")
    blk_mean = torch.full((B * seq_stride,), -9.0, device="cuda")
    out = torch.empty((B, Hq, d), device="cuda")
    probs = torch.full((B, Hq, c["stride"]), -7.0, device="cuda")
    cum0 = torch.rand((B, Hkv, c["stride"]), device="cuda")
    cum = cum0.clone()
    prev = K.set_sync_wait_us(wait_us) if wait_us is not None else None
    try:
        layer = 1                                                # write the second stacked layer
        off = layer * Hkv * head_stride
        K.decode_attn_scores_agg(kv, c["q"], Hq, c["scale"], out, None, probs, cum, 0.5, bs,
                                 blk_max[off:], blk_mean[off:], head_stride, seq_stride)
        torch.cuda.synchronize()
    finally:
        if prev is not None:
            K.set_sync_wait_us(prev)
    bm = blk_max.view(-1)
    bn = blk_mean.view(-1)
    for b in range(B):
        L = lengths[b]
        r = _oracle(c, b)
        assert max_rel(f64(probs[b, :, :L]), r["probs"]) < SCORE_TOL
        cum_ref = O.accumulate(f64(cum0[b, :, :L]), r["probs"], decay=0.5)
        assert max_rel(f64(cum[b, :, :L]), cum_ref) < SCORE_TOL
        want_max, want_mean = O.block_aggregate(cum_ref, L, bs)
        nb = -(-L // bs)
        for h in range(Hkv):
            base = b * seq_stride + off + h * head_stride
            assert max_rel(f64(bm[base:base + nb]), want_max[h]) < SCORE_TOL
            assert max_rel(f64(bn[base:base + nb]), want_mean[h]) < SCORE_TOL
            assert (bm[base + nb:base + head_stride] == -9.0).all()
        # the other stacked layer and the padding are untouched
        assert (bm[b * seq_stride:b * seq_stride + off] == -9.0).all()
