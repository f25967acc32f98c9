"""Run-to-run determinism: every path other than the decode pass (tested in
test_gpu_decode.py) gives the same bits when run twice on the same inputs,
with workspaces filled with different junk before each run.  None of these
kernels sums floats through atomics, and the selections break ties by
position, so any difference would be a race."""
import math

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _K():
    import attention_score_guided_amd as K
    return K


def _junk(nbytes, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randint(0, 256, (max(nbytes, 256),), dtype=torch.uint8, device="cuda", generator=g)


def _twice(run):
    """run(seed) returns a list of tensors; both runs must agree bit for bit."""
    a = [t.clone() for t in run(1)]
    b = [t.clone() for t in run(2)]
    torch.cuda.synchronize()
    for i, (x, y) in enumerate(zip(a, b)):
        assert torch.equal(x, y), f"output {i} differs between two runs"


def test_vote_sparse_quest_indexer_deterministic():
    K = _K()
    B, Hq, Hkv, d, P, L, W = 2, 8, 2, 128, 16, 24000, 32
    g = synth.generator(101, "cuda")
    bt, n_pages = synth.shuffled_block_table(B, L + 1, P, g, "cuda")
    kp = synth.normal((n_pages, Hkv, P, d), g, torch.bfloat16, "cuda")
    vp = synth.normal((n_pages, Hkv, P, d), g, torch.bfloat16, "cuda")
    kip = synth.normal((n_pages, 1, P, 64), g, torch.bfloat16, "cuda")
    lens = torch.tensor([L, L - 1234], dtype=torch.int32, device="cuda")
    kv = K.PagedKV(kp, vp, bt, lens, P, L + 1)
    kv_k = K.PagedKV(kp, None, bt, lens, P, L + 1)
    kvi = K.PagedKV(kip, None, bt, lens, P, L + 1)
    kvi8 = K.PagedKV(kip.to(torch.float8_e4m3fn), None, bt, lens, P, L + 1)
    q_win = synth.normal((B, Hq, W, d), g, torch.bfloat16, "cuda")
    q = synth.normal((B, Hq, d), g, torch.bfloat16, "cuda")
    qi = synth.normal((B, Hq, 64), g, torch.bfloat16, "cuda")
    qi8 = qi.to(torch.float8_e4m3fn)
    scale = 1 / math.sqrt(d)

    def vote(seed):
        votes = torch.zeros((B, Hkv, L + 1), device="cuda")
        K.snapkv_vote(kv_k, q_win, Hq, W, 7, scale, K.REDUCE_SUM, votes,
                      workspace=_junk(K.snapkv_workspace_bytes(kv_k, Hq, W), seed))
        return [votes]
    _twice(vote)

    k = 2048
    for kvx, qx in ((kvi, qi), (kvi8, qi8)):
        def topk_and_attend(seed, kvx=kvx, qx=qx):
            keep = torch.full((B * Hq, k), -1, dtype=torch.int32, device="cuda")
            cnt = torch.zeros((B * Hq,), dtype=torch.int32, device="cuda")
            K.indexer_topk(kvx, qx, Hq, 1.0, k, keep, cnt, workspace=_junk(K.indexer_topk_workspace_bytes(kvx, Hq, k), seed))
            out = torch.zeros((B, Hq, d), device="cuda")
            K.sparse_attn(kv, q, Hq, keep.view(B, Hq, k), cnt.view(B, Hq), k, scale, out,
                          workspace=_junk(K.sparse_workspace_bytes(B, Hq, d, k), seed))
            return [keep, cnt, out]
        _twice(topk_and_attend)

    summary = torch.empty((n_pages, Hkv, 2, d), dtype=torch.bfloat16, device="cuda")
    K.quest_summarize(kv_k, summary)

    def quest(seed):
        QP = 64
        qidx = torch.full((B, Hq, QP * P + P - 1), -1, dtype=torch.int32, device="cuda")
        qcnt = torch.zeros((B, Hq), dtype=torch.int32, device="cuda")
        K.quest_select(kv_k, summary, q, Hq, QP, qidx, qcnt,
                       workspace=_junk(K.quest_workspace_bytes(kv_k, Hq, QP), seed))
        return [qidx, qcnt]
    _twice(quest)


def test_h2o_step_deterministic():
    K = _K()
    B, Hq, Hkv, d, P, L0 = 2, 8, 2, 128, 16, 5000
    sinks, window, budget = 4, 64, 900
    g = synth.generator(102, "cuda")
    bt, n_pages = synth.shuffled_block_table(B, L0 + 2, P, g, "cuda")
    kp = synth.normal((n_pages, Hkv, P, d), g, torch.bfloat16, "cuda")
    vp = synth.normal((n_pages, Hkv, P, d), g, torch.bfloat16, "cuda")
    q = synth.normal((B, Hq, d), g, torch.bfloat16, "cuda")
    kv = K.PagedKV(kp, vp, bt, torch.full((B,), L0 + 1, dtype=torch.int32, device="cuda"), P, L0 + 2)
    stride = L0 + 16
    # lists longer than the budget: the first step sheds many slots (the general path)
    slots0 = torch.arange(L0, dtype=torch.int32, device="cuda").repeat(B, Hkv, 1)
    slots0 = torch.cat([slots0, torch.zeros((B, Hkv, stride - L0), dtype=torch.int32, device="cuda")], dim=-1)
    cum0 = torch.rand((B, Hkv, stride), generator=torch.Generator(device="cuda").manual_seed(3), device="cuda")
    cnt0 = torch.full((B, Hkv), L0, dtype=torch.int32, device="cuda")

    def step(seed):
        sl, cm, cn = slots0.clone(), cum0.clone(), cnt0.clone()
        out = torch.zeros((B, Hq, d), device="cuda")
        probs = torch.zeros((B, Hq, stride), device="cuda")
        K.h2o_step(kv, q, Hq, 1 / math.sqrt(d), sl, cm, cn, sinks, window, budget, out, probs=probs,
                   workspace=_junk(K.h2o_workspace_bytes(kv, Hq, stride, sinks, window, budget), seed))
        return [sl, cm, cn, out, probs]
    _twice(step)
