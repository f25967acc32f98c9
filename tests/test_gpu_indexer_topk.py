"""GPU parity of kvsel_indexer_topk, bf16 and FP8 E4M3 ([LONGCTX] "sparse attention" experiment:
the indexer scores every cached key and each query keeps its top 2048).

The fused call never writes the scores, so it is checked two ways:
  * bit-exact against kvsel_decode_attn_scores (EMIT_LOGITS) followed by
    kvsel_select_keep (ROWS, sinks 0, window 0, budget k) on the same inputs:
    every row's keep list and count, in every case;
  * end to end against the oracle's selection on its own float64 scores, on
    sampled rows: any difference must be a swap between scores within 1e-6
    of the cut (the worst gap is printed).
Cases: the 128K sparse-step configuration the benchmark times (B=4, 32 query
heads on one d=64 indexer head, L=131073, k=2048), ragged rows, d=128 with
G=4, G=32, rows that keep everything (k >= L_b), a row too short for its
sample to bound the cut (every position stored), the shapes that take the
materialised path (short rows, k > L/8), and both fallbacks of the fused
path: massive ties (every score equal, so more than 16384 keys reach the
sampled bound) and a bound set too high by keys that score high only at the
sampled positions.  Workspaces are filled with junk first: nothing in them
may be read before it is written."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.parity_util import f64, keep_swap_gap, logical_kv_rows, note

pytestmark = pytest.mark.gpu


def _K():
    import attention_score_guided_amd as K
    return K


def _cache(B, Hkv, d, lens, P, seed, kfn=None):
    """Paged bf16 indexer cache (shuffled pages, N(0,1) keys unless kfn gives
    the logical keys [B][Hkv][cap][d]) and its PagedKV."""
    K = _K()
    g = synth.generator(seed, "cuda")
    cap = max(lens)
    bt, n_pages = synth.shuffled_block_table(B, cap, P, g, "cuda")
    if kfn is None:
        kp = synth.normal((n_pages, Hkv, P, d), g, torch.bfloat16, "cuda")
    else:
        logical = kfn(g, cap).to(torch.bfloat16)
        kp = torch.zeros((n_pages, Hkv, P, d), dtype=torch.bfloat16, device="cuda")
        for b in range(B):
            for c in range(Hkv):
                synth.write_positions(kp[:, c:c + 1], bt[b], 0, logical[b, c:c + 1])
    lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
    return K.PagedKV(kp, None, bt, lt, P, cap), kp, bt


def _junk(nbytes):
    return torch.randint(0, 256, (max(nbytes, 256),), dtype=torch.uint8, device="cuda")


def _unfused(kv, q, Hq, scale, k):
    K = _K()
    B, cap = q.shape[0], kv.desc.max_seq_len
    stride = -(-cap // 4) * 4
    scores = torch.empty((B, Hq, stride), device="cuda")
    K.decode_attn_scores(kv, q, Hq, scale, None, None, scores, K.EMIT_LOGITS)
    rows = scores.view(B * Hq, stride)
    lens = kv.seq_lens.repeat_interleave(Hq).to(torch.int32)
    kk = min(k, cap)
    keep = torch.full((B * Hq, kk), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B * Hq,), -7, dtype=torch.int32, device="cuda")
    K.select_keep(rows, lens, cap, 0, 0, None, k, keep, cnt)
    return keep, cnt, scores


def _fused(kv, q, Hq, scale, k):
    K = _K()
    B, cap = q.shape[0], kv.desc.max_seq_len
    kk = min(k, cap)
    keep = torch.full((B * Hq, kk), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B * Hq,), -7, dtype=torch.int32, device="cuda")
    ws = _junk(K.indexer_topk_workspace_bytes(kv, Hq, k))
    K.indexer_topk(kv, q, Hq, scale, k, keep, cnt, workspace=ws)
    return keep, cnt


def _same_sets(kf, cf, ku, cu):
    assert torch.equal(cf, cu), "counts differ from the unfused path"
    for r in range(cf.numel()):
        n = int(cf[r])
        assert torch.equal(kf[r, :n], ku[r, :n]), f"row {r}: keep list differs from the unfused path"


def _oracle_rows(kp, bt, q, scale, lens, Hq, G, k, rows):
    """End-to-end check of the fused sets on a few rows against the oracle's
    selection on float64 scores."""
    for r, got in rows:
        b, h = r // Hq, r % Hq
        L = lens[b]
        KI, _ = logical_kv_rows(kp, None, bt, b, h // G, L)
        want_s = O.indexer_scores(f64(q[b, h])[None, :], KI[0])[0] * scale
        e2e = O.select_keep(want_s, L, 0, 0, k)
        gap = keep_swap_gap(got, e2e, want_s, L)
        note(f"  row b={b} h={h}: {len(set(got.tolist()) ^ set(e2e.tolist()))} differing from the oracle's "
             f"set, worst gap {gap:.2e}")


def test_indexer_topk_128k_sparse_step():
    """The benchmark's sparse-step selection at full size: every row equal to
    the unfused path, sampled rows against the oracle."""
    K = _K()
    L, B, Hq = 131072, 4, 32
    cfg = synth.long_context_128k(seq_len=L, sparse_steps=1, device="cuda")
    kit = cfg["kv_index"]
    lens = kit.seq_lens.clone() + 1
    kvi = K.PagedKV(kit.k_pages, None, kit.block_table, lens, 16, L + 1)
    q = cfg["qi_dec"][0]
    kf, cf = _fused(kvi, q, Hq, 1.0, 2048)
    ku, cu, _ = _unfused(kvi, q, Hq, 1.0, 2048)
    torch.cuda.synchronize()
    _same_sets(kf, cf, ku, cu)
    assert int(cf.min()) == 2048
    rows = [(r, kf[r, :int(cf[r])].cpu().numpy()) for r in (0, 2 * Hq + 17, 3 * Hq + 31)]
    _oracle_rows(kit.k_pages, kit.block_table, q, 1.0, [L + 1] * B, Hq, Hq, 2048, rows)


@pytest.mark.parametrize("B,Hkv,Hq,d,lens,k,P,scale", [
    (2, 1, 8, 64, [40000, 23457], 2048, 16, 1.0),        # fused, ragged rows
    (2, 2, 8, 128, [20000, 16391], 1024, 32, 0.125),     # fused, d=128, G=4
    (1, 1, 32, 64, [70001], 2048, 64, 1.0),              # fused, G=32 (two column tiles)
    (3, 1, 16, 64, [17000, 1500, 2048], 2048, 16, 1.0),  # fused; two rows keep everything
    (2, 1, 8, 64, [20000, 2100], 2048, 16, 1.0),         # fused; a short row's sample is below k_lo (bound 0)
    (2, 1, 4, 64, [4000, 3001], 512, 16, 1.0),           # short rows: materialised logits
    (1, 1, 8, 64, [20000], 6144, 16, 1.0),               # k > L / 8: materialised logits
])
def test_indexer_topk_shapes(B, Hkv, Hq, d, lens, k, P, scale):
    note(f"indexer top-{k}: B={B} H_kv={Hkv} H_q={Hq} d={d} lens={lens} page={P}")
    kv, kp, bt = _cache(B, Hkv, d, lens, P, seed=11 + B + d)
    g = synth.generator(5 + Hq, "cuda")
    q = synth.normal((B, Hq, d), g, torch.bfloat16, "cuda")
    kf, cf = _fused(kv, q, Hq, scale, k)
    ku, cu, _ = _unfused(kv, q, Hq, scale, k)
    torch.cuda.synchronize()
    _same_sets(kf, cf, ku, cu)
    want_counts = [min(k, lens[r // Hq]) for r in range(B * Hq)]
    assert cf.cpu().tolist() == want_counts
    picks = sorted({0, B * Hq - 1, (B // 2) * Hq + Hq // 2})
    rows = [(r, kf[r, :int(cf[r])].cpu().numpy()) for r in picks]
    _oracle_rows(kp, bt, q, scale, lens, Hq, Hq // Hkv, k, rows)


def test_indexer_topk_fallback_ties():
    """Every key equal (zero keys): every middle position reaches the sampled
    bound, more than the final pass holds, so each row falls back to its
    recomputed scores; ties resolve to the lowest positions."""
    B, Hq, L, k = 2, 8, 20000, 2048
    kv, _, _ = _cache(B, 1, 64, [L, L - 3], 16, seed=3,
                      kfn=lambda g, cap: torch.zeros((B, 1, cap, 64), device="cuda"))
    q = synth.normal((B, Hq, 64), synth.generator(9, "cuda"), torch.bfloat16, "cuda")
    kf, cf = _fused(kv, q, Hq, 1.0, k)
    ku, cu, _ = _unfused(kv, q, Hq, 1.0, k)
    torch.cuda.synchronize()
    _same_sets(kf, cf, ku, cu)
    expect = torch.arange(k, dtype=torch.int32, device="cuda")
    for r in range(B * Hq):
        assert torch.equal(kf[r, :k], expect)


def test_indexer_topk_fallback_bound_too_high():
    """Keys that score high only at the sampled positions (the first 16 of
    every 256) put the sampled bound above the cut: fewer than k keys reach
    it, so each row falls back to its recomputed scores."""
    B, Hq, L, k, d = 1, 2, 30000, 2048, 64
    g0 = synth.generator(21, "cuda")
    q = synth.normal((B, Hq, d), g0, torch.bfloat16, "cuda")
    qdir = q[0, 0].float()
    qdir = qdir / qdir.norm()     # head 0 scores the planted direction positively

    def keys(g, cap):
        kl = 0.05 * synth.normal((B, 1, cap, d), g, torch.float32, "cuda")
        pos = torch.arange(cap, device="cuda")
        hot = (pos % 256) < 16
        amp = 2.0 + torch.rand(cap, generator=g, device="cuda")
        kl[0, 0, hot] += amp[hot, None] * qdir[None, :]
        kl[0, 0, ~hot] += 0.5 * amp[~hot, None] * qdir[None, :]
        return kl

    kv, kp, bt = _cache(B, 1, d, [L], 16, seed=4, kfn=keys)
    kf, cf = _fused(kv, q, Hq, 1.0, k)
    ku, cu, scores = _unfused(kv, q, Hq, 1.0, k)
    torch.cuda.synchronize()
    _same_sets(kf, cf, ku, cu)
    # the premise (head 0): the sampled positions hold the largest scores but
    # fewer than k of them, so the k largest reach past them
    s0 = scores[0, 0, :L].float()
    top = torch.topk(s0, k).indices
    hot = int(((top % 256) < 16).sum())
    assert hot == int(((torch.arange(L, device="cuda") % 256) < 16).sum()) and hot < k
    rows = [(r, kf[r, :int(cf[r])].cpu().numpy()) for r in (0, Hq - 1)]
    _oracle_rows(kp, bt, q, 1.0, [L], Hq, Hq, k, rows)


# ---- FP8 E4M3 indexer (keys and queries stored as E4M3) ---------------------
# The fused call scores with the FP8 matrix-core chain of
# kvsel_indexer_scores_fp8 (same channels per k-step, same order), so its sets
# equal kvsel_indexer_scores_fp8 + kvsel_select_keep bit for bit; sampled rows
# are checked against the oracle's selection on float64 scores of the decoded
# E4M3 values.  The FP8 matrix cores do not sum their products like a chain of
# fp32 adds (errors up to ~3e-5 of sum_d |q_d k_d| were measured for the FP8
# indexer), so a swap with the oracle's set is allowed where both keys' oracle
# scores lie within the FP8 score tolerance, 1e-4 of that sum, of the cut.
FP8_SCORE_TOL = 1e-4


def _fp8_swaps_ok(got, want, scores, err_scale):
    """Equal sets, or every differing key's oracle score within FP8_SCORE_TOL
    of its error scale from the oracle's cut; returns the worst such ratio."""
    got, want = set(int(x) for x in got), set(int(x) for x in want)
    assert len(got) == len(want), f"keep sets differ in size: {len(got)} vs {len(want)}"
    diff = sorted(got ^ want)
    if not diff:
        return 0.0
    tau = min(scores[j] for j in want)
    worst = max(abs(scores[j] - tau) / err_scale[j] for j in diff)
    assert worst <= FP8_SCORE_TOL, (f"{len(diff)} differing positions, worst |s - tau| / sum|q k| {worst:.3e} "
                                    f"> {FP8_SCORE_TOL:g} (tau {tau:.9g}; positions {diff[:8]})")
    return worst

def _fp8_from(t):
    return t.to(torch.float8_e4m3fn)


def _unfused_fp8(kv, q, Hq, scale, k):
    K = _K()
    B, cap = q.shape[0], kv.desc.max_seq_len
    stride = -(-cap // 4) * 4
    scores = torch.empty((B, Hq, stride), device="cuda")
    K.indexer_scores_fp8(kv, q, Hq, scale, scores)
    rows = scores.view(B * Hq, stride)
    lens = kv.seq_lens.repeat_interleave(Hq).to(torch.int32)
    kk = min(k, cap)
    keep = torch.full((B * Hq, kk), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B * Hq,), -7, dtype=torch.int32, device="cuda")
    K.select_keep(rows, lens, cap, 0, 0, None, k, keep, cnt)
    return keep, cnt


def _oracle_rows_fp8(kp, bt, q, scale, lens, Hq, G, k, rows):
    P = kp.shape[2]
    for r, got in rows:
        b, h = r // Hq, r % Hq
        L = lens[b]
        n_pg = -(-L // P)
        pages = bt[b, :n_pg].long()
        kbits = kp[pages, h // G].contiguous().view(torch.uint8).cpu().numpy()     # [n_pg][P][d]
        KI = O.fp8_e4m3_bits_to_f64(kbits).reshape(n_pg * P, -1)[:L]
        qv = O.fp8_e4m3_bits_to_f64(q[b, h].contiguous().view(torch.uint8).cpu().numpy())
        want_s = O.indexer_scores(qv[None, :], KI)[0] * scale
        err_scale = np.maximum(scale * (np.abs(KI) @ np.abs(qv)), 1e-30)
        e2e = O.select_keep(want_s, L, 0, 0, k)
        gap = _fp8_swaps_ok(got, e2e, want_s, err_scale)
        note(f"  fp8 row b={b} h={h}: {len(set(got.tolist()) ^ set(e2e.tolist()))} differing from the oracle's "
             f"set, worst |s - tau| / sum|q k| {gap:.2e}")


def test_indexer_topk_fp8_128k_sparse_step():
    """The 128K sparse step's indexer in FP8 at full size (B=4, 32 heads on
    one d=64 indexer head, L=131073, top-2048)."""
    K = _K()
    L, B, Hq = 131072, 4, 32
    cfg = synth.long_context_128k(seq_len=L, sparse_steps=1, device="cuda")
    kit = cfg["kv_index"]
    lens = kit.seq_lens.clone() + 1
    kp8 = _fp8_from(kit.k_pages)
    kvi = K.PagedKV(kp8, None, kit.block_table, lens, 16, L + 1)
    q = _fp8_from(cfg["qi_dec"][0])
    kf, cf = _fused(kvi, q, Hq, 1.0, 2048)
    ku, cu = _unfused_fp8(kvi, q, Hq, 1.0, 2048)
    torch.cuda.synchronize()
    _same_sets(kf, cf, ku, cu)
    assert int(cf.min()) == 2048
    rows = [(r, kf[r, :int(cf[r])].cpu().numpy()) for r in (0, Hq + 5, 3 * Hq + 31)]
    _oracle_rows_fp8(kp8, kit.block_table, q, 1.0, [L + 1] * B, Hq, Hq, 2048, rows)


@pytest.mark.parametrize("B,Hkv,Hq,d,lens,k,P,scale", [
    (2, 1, 8, 64, [40000, 23457], 2048, 16, 1.0),        # fused, ragged rows
    (2, 2, 8, 128, [20000, 16391], 1024, 32, 0.125),     # fused, d=128, G=4
    (1, 1, 32, 64, [70001], 2048, 64, 1.0),              # fused, G=32 (two column tiles)
    (3, 1, 16, 64, [17000, 1500, 2048], 2048, 16, 1.0),  # fused; two rows keep everything
    (2, 1, 8, 64, [20000, 2100], 2048, 16, 1.0),         # fused; a short row's sample is below k_lo (bound 0)
    (2, 1, 4, 64, [4000, 3001], 512, 16, 1.0),           # short rows: materialised FP8 scores
    (1, 1, 8, 64, [20000], 6144, 16, 1.0),               # k > L / 8: materialised FP8 scores
])
def test_indexer_topk_fp8_shapes(B, Hkv, Hq, d, lens, k, P, scale):
    note(f"fp8 indexer top-{k}: B={B} H_kv={Hkv} H_q={Hq} d={d} lens={lens} page={P}")
    K = _K()
    g = synth.generator(31 + B + d, "cuda")
    cap = max(lens)
    bt, n_pages = synth.shuffled_block_table(B, cap, P, g, "cuda")
    kp = _fp8_from(2.0 * synth.normal((n_pages, Hkv, P, d), g, torch.float32, "cuda"))
    kv = K.PagedKV(kp, None, bt, torch.tensor(lens, dtype=torch.int32, device="cuda"), P, cap)
    q = _fp8_from(2.0 * synth.normal((B, Hq, d), g, torch.float32, "cuda"))
    kf, cf = _fused(kv, q, Hq, scale, k)
    ku, cu = _unfused_fp8(kv, q, Hq, scale, k)
    torch.cuda.synchronize()
    _same_sets(kf, cf, ku, cu)
    assert cf.cpu().tolist() == [min(k, lens[r // Hq]) for r in range(B * Hq)]
    picks = sorted({0, B * Hq - 1, (B // 2) * Hq + Hq // 2})
    rows = [(r, kf[r, :int(cf[r])].cpu().numpy()) for r in picks]
    _oracle_rows_fp8(kp, bt, q, scale, lens, Hq, Hq // Hkv, k, rows)


def test_indexer_topk_mixed_dtypes_rejected():
    """bf16 queries on FP8 pages are refused before any launch."""
    K = _K()
    g = synth.generator(5, "cuda")
    bt, n_pages = synth.shuffled_block_table(1, 4096, 16, g, "cuda")
    kp = _fp8_from(synth.normal((n_pages, 1, 16, 64), g, torch.float32, "cuda"))
    kv = K.PagedKV(kp, None, bt, torch.tensor([4096], dtype=torch.int32, device="cuda"), 16, 4096)
    q = synth.normal((1, 8, 64), g, torch.bfloat16, "cuda")
    keep = torch.empty((8, 256), dtype=torch.int32, device="cuda")
    cnt = torch.empty((8,), dtype=torch.int32, device="cuda")
    with pytest.raises(TypeError):
        K.indexer_topk(kv, q, 8, 1.0, 256, keep, cnt)


def test_indexer_topk_fp8_fallback_ties():
    """FP8 keys all zero: every score is 0, more keys reach the sampled bound
    than the final pass holds, and each row is selected from its scores
    recomputed with the FP8 chain; ties resolve to the lowest positions."""
    K = _K()
    B, Hq, L, k = 2, 8, 20000, 2048
    g = synth.generator(3, "cuda")
    bt, n_pages = synth.shuffled_block_table(B, L, 16, g, "cuda")
    kp = torch.zeros((n_pages, 1, 16, 64), device="cuda").to(torch.float8_e4m3fn)
    kv = K.PagedKV(kp, None, bt, torch.tensor([L, L - 3], dtype=torch.int32, device="cuda"), 16, L)
    q = _fp8_from(synth.normal((B, Hq, 64), g, torch.float32, "cuda"))
    kf, cf = _fused(kv, q, Hq, 1.0, k)
    ku, cu = _unfused_fp8(kv, q, Hq, 1.0, k)
    torch.cuda.synchronize()
    _same_sets(kf, cf, ku, cu)
    expect = torch.arange(k, dtype=torch.int32, device="cuda")
    for r in range(B * Hq):
        assert torch.equal(kf[r, :k], expect)


def test_indexer_topk_fp8_fallback_bound_too_high():
    """FP8 keys that score high only at the sampled positions (the first 16
    of every 256): fewer than k keys reach the sampled bound, so each row
    falls back to its FP8 scores recomputed in the final pass."""
    K = _K()
    B, Hq, L, k, d = 1, 2, 30000, 2048, 64
    g = synth.generator(21, "cuda")
    q32 = synth.normal((B, Hq, d), g, torch.float32, "cuda")
    q = _fp8_from(q32)
    qdir = q.float()[0, 0]
    qdir = qdir / qdir.norm()
    bt, n_pages = synth.shuffled_block_table(B, L, 16, g, "cuda")
    kl = 0.05 * synth.normal((L, d), g, torch.float32, "cuda")
    pos = torch.arange(L, device="cuda")
    hot = (pos % 256) < 16
    amp = 2.0 + torch.rand(L, generator=g, device="cuda")
    kl[hot] += amp[hot, None] * qdir[None, :]
    kl[~hot] += 0.5 * amp[~hot, None] * qdir[None, :]
    kp = torch.zeros((n_pages, 1, 16, d), device="cuda")
    synth.write_positions(kp, bt[0], 0, kl[None, :, :])
    kp = kp.to(torch.float8_e4m3fn)
    kv = K.PagedKV(kp, None, bt, torch.tensor([L], dtype=torch.int32, device="cuda"), 16, L)
    kf, cf = _fused(kv, q, Hq, 1.0, k)
    ku, cu = _unfused_fp8(kv, q, Hq, 1.0, k)
    torch.cuda.synchronize()
    _same_sets(kf, cf, ku, cu)
    # the premise on the FP8 scores of head 0: the k largest reach past the sampled positions
    stride = -(-L // 4) * 4
    sc = torch.empty((B, Hq, stride), device="cuda")
    K.indexer_scores_fp8(kv, q, Hq, 1.0, sc)
    top = torch.topk(sc[0, 0, :L], k).indices
    n_hot = int(hot.sum())
    assert int(((top % 256) < 16).sum()) == n_hot and n_hot < k
    rows = [(r, kf[r, :int(cf[r])].cpu().numpy()) for r in (0, Hq - 1)]
    _oracle_rows_fp8(kp, bt, q, 1.0, [L], Hq, Hq, k, rows)
