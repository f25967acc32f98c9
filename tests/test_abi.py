"""The C-ABI library loads, exports every declared symbol and rejects bad
arguments before touching HIP.  CPU only: no call here launches a kernel."""
import ctypes
import re

import pytest

import attention_score_guided_amd as K
from attention_score_guided_amd import _lib

HEADER = "include/kvsel.h"


def _declared_functions():
    import os
    src = open(os.path.join(os.path.dirname(__file__), "..", HEADER)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvsel_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    lib = K.library()
    decl = _declared_functions()
    assert len(decl) >= 11
    for name in decl:
        assert hasattr(lib, name), name
    assert sorted(decl) == sorted(K.EXPORTED)


def test_status_strings():
    lib = K.library()
    assert lib.kvsel_status_string(0) == b"KVSEL_OK"
    assert lib.kvsel_status_string(-1) == b"KVSEL_ERR_INVALID"
    assert lib.kvsel_status_string(-3) == b"KVSEL_ERR_WORKSPACE"


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _kv(**over):
    d = dict(k_pages=FAKE, v_pages=FAKE, block_table=FAKE, seq_lens=FAKE, num_seqs=2, num_kv_heads=8,
             head_dim=128, page_size=16, max_pages_per_seq=64, max_seq_len=1024, dtype=K.KVSEL_BF16)
    d.update(over)
    return K.PagedKVDesc(**d)


def _decode(kv, hq=32, probs=FAKE, probs_stride=1024, emit=0, cum=None, cum_stride=1024, ws=FAKE,
            wsb=1 << 30, out=FAKE, q=FAKE):
    lib = K.library()
    return lib.kvsel_decode_attn_scores(ctypes.byref(kv), q, hq, 0.1, out, None, probs, probs_stride,
                                        emit, cum, cum_stride, 1.0, ws, wsb, None)


@pytest.mark.parametrize("over,hq,kw,status", [
    ({}, 32, dict(q=None), K.KVSEL_ERR_INVALID),
    ({"k_pages": None}, 32, {}, K.KVSEL_ERR_INVALID),
    ({"v_pages": None}, 32, {}, K.KVSEL_ERR_INVALID),          # out needs V
    ({"num_seqs": 0}, 32, {}, K.KVSEL_ERR_INVALID),
    ({}, 30, {}, K.KVSEL_ERR_INVALID),                           # 30 % 8 != 0
    ({}, 32, dict(probs_stride=1000), K.KVSEL_ERR_INVALID),
    ({}, 32, dict(cum=FAKE, cum_stride=10), K.KVSEL_ERR_INVALID),
    ({"max_pages_per_seq": 10}, 32, {}, K.KVSEL_ERR_INVALID),
    ({}, 32, dict(emit=7), K.KVSEL_ERR_INVALID),
    ({"head_dim": 96}, 32, {}, K.KVSEL_ERR_UNSUPPORTED),
    ({"dtype": 5}, 32, {}, K.KVSEL_ERR_UNSUPPORTED),
    ({"page_size": 8, "max_pages_per_seq": 128}, 32, {}, K.KVSEL_ERR_UNSUPPORTED),
    ({"page_size": 48}, 32, {}, K.KVSEL_ERR_UNSUPPORTED),
    ({}, 32, dict(emit=1, cum=FAKE), K.KVSEL_ERR_UNSUPPORTED),   # cum needs probabilities
    ({"num_kv_heads": 4}, 24, {}, K.KVSEL_ERR_UNSUPPORTED),      # G = 6
    ({}, 32, dict(ws=None), K.KVSEL_ERR_WORKSPACE),
    ({}, 32, dict(wsb=16), K.KVSEL_ERR_WORKSPACE),
])
def test_decode_validation(over, hq, kw, status):
    assert _decode(_kv(**over), hq=hq, **kw) == status
    assert K.library().kvsel_last_error() != b""


def test_workspace_query():
    lib = K.library()
    kv = _kv()
    a = lib.kvsel_decode_workspace_bytes(ctypes.byref(kv), 32, 1)
    b = lib.kvsel_decode_workspace_bytes(ctypes.byref(kv), 32, 0)
    assert a > 0 and b >= a + 2 * 32 * 1024 * 4
    assert lib.kvsel_decode_workspace_bytes(ctypes.byref(_kv(head_dim=96)), 32, 1) == 0


def test_accumulate_and_aggregate_validation():
    lib = K.library()
    assert lib.kvsel_accumulate(None, 8, FAKE, 1, 4, 1, 8, 1.0, FAKE, 8, None) == K.KVSEL_ERR_INVALID
    assert lib.kvsel_accumulate(FAKE, 8, FAKE, 1, 6, 4, 8, 1.0, FAKE, 8, None) == K.KVSEL_ERR_INVALID
    assert lib.kvsel_accumulate(FAKE, 4, FAKE, 1, 4, 1, 8, 1.0, FAKE, 8, None) == K.KVSEL_ERR_INVALID
    agg = lib.kvsel_block_aggregate
    assert agg(FAKE, 64, FAKE, 1, 1, 64, 16, 0, 0, None, None, 4, None) == K.KVSEL_ERR_INVALID
    assert agg(FAKE, 64, FAKE, 1, 1, 64, 16, 0, 0, FAKE, None, 3, None) == K.KVSEL_ERR_INVALID
    assert agg(FAKE, 64, FAKE, 1, 1, 64, 16, 2, 0, FAKE, None, 4, None) == K.KVSEL_ERR_INVALID
    assert agg(FAKE, 63, FAKE, 1, 1, 64, 16, 0, 0, FAKE, None, 4, None) == K.KVSEL_ERR_INVALID
    assert agg(FAKE, 64, FAKE, 1, 1, 64, 0, 0, 0, FAKE, None, 4, None) == K.KVSEL_ERR_INVALID


def test_select_validation():
    lib = K.library()
    sel = lib.kvsel_select_keep
    ok = dict(scores=FAKE, stride=100, lengths=FAKE, rows=4, max_len=100, sinks=4, window=8,
              budgets=None, max_budget=20, mode=0, gb=0, out=FAKE, out_stride=20, cnt=FAKE,
              ws=None, wsb=0)

    def call(**kw):
        a = dict(ok, **kw)
        return sel(a["scores"], a["stride"], a["lengths"], a["rows"], a["max_len"], a["sinks"],
                   a["window"], a["budgets"], a["max_budget"], a["mode"], a["gb"], a["out"],
                   a["out_stride"], a["cnt"], a["ws"], a["wsb"], None)
    assert call(scores=None) == K.KVSEL_ERR_INVALID
    assert call(rows=0) == K.KVSEL_ERR_INVALID
    assert call(stride=99) == K.KVSEL_ERR_INVALID
    assert call(sinks=-1) == K.KVSEL_ERR_INVALID
    assert call(out_stride=19) == K.KVSEL_ERR_INVALID
    assert call(mode=3) == K.KVSEL_ERR_INVALID
    assert call(mode=1) == K.KVSEL_ERR_INVALID                      # sinks/window in GLOBAL
    g = dict(mode=1, sinks=0, window=0, out_stride=100)
    assert call(**g, ws=None) == K.KVSEL_ERR_WORKSPACE
    assert call(**dict(g, max_len=9000, stride=9000, out_stride=9000)) == K.KVSEL_ERR_UNSUPPORTED
    assert lib.kvsel_select_workspace_bytes(4, 100, 1) >= 4 * 100 * 8
    assert lib.kvsel_select_workspace_bytes(4, 100, 0) == 0


def test_sparse_validation():
    lib = K.library()
    kv = _kv()
    def call(hq=32, idx=FAKE, cnt=FAKE, idx_heads=32, max_count=10, stride=16, out=FAKE, ws=FAKE, wsb=1 << 30, kvd=kv):
        return lib.kvsel_sparse_attn(ctypes.byref(kvd), FAKE, hq, idx, stride, cnt, idx_heads, max_count, 0.1,
                                     out, None, ws, wsb, None)
    assert call(idx=None) == K.KVSEL_ERR_INVALID
    assert call(out=None) == K.KVSEL_ERR_INVALID
    assert call(idx_heads=5) == K.KVSEL_ERR_INVALID
    assert call(max_count=20) == K.KVSEL_ERR_INVALID
    assert call(kvd=_kv(v_pages=None)) == K.KVSEL_ERR_INVALID
    assert call(hq=96, idx_heads=8) == K.KVSEL_ERR_UNSUPPORTED     # shared sets with G = 12
    assert call(ws=None) == K.KVSEL_ERR_WORKSPACE
    assert lib.kvsel_sparse_workspace_bytes(4, 32, 128, 2048) >= 4 * 32 * 8 * 128 * 4


def test_snapkv_validation():
    lib = K.library()
    def call(kvd=None, window=32, pool=7, red=1, votes=FAKE, stride=1024, ws=FAKE, wsb=1 << 30):
        kvd = kvd or _kv()
        return lib.kvsel_snapkv_vote(ctypes.byref(kvd), FAKE, 32, window, pool, 0.1, red, votes, stride, ws, wsb, None)
    assert call(votes=None) == K.KVSEL_ERR_INVALID
    assert call(window=0) == K.KVSEL_ERR_INVALID
    assert call(window=1024) == K.KVSEL_ERR_INVALID
    assert call(pool=6) == K.KVSEL_ERR_INVALID
    assert call(red=3) == K.KVSEL_ERR_INVALID
    assert call(stride=100) == K.KVSEL_ERR_INVALID
    assert call(kvd=_kv(dtype=K.KVSEL_F32)) == K.KVSEL_ERR_UNSUPPORTED
    assert call(window=65) == K.KVSEL_ERR_UNSUPPORTED
    assert call(ws=None) == K.KVSEL_ERR_WORKSPACE
    # chunk partials (max, sum) of every window row plus the per-row lse
    assert lib.kvsel_snapkv_workspace_bytes(ctypes.byref(_kv()), 32, 32) >= 2 * 32 * 32 * 4 * 8


def test_sync_wait_bound_setter():
    prev = K.set_sync_wait_us(7)
    try:
        assert prev >= 0
        assert K.set_sync_wait_us(0) == 7
        with pytest.raises(K.KvselError):
            K.set_sync_wait_us(-1)
        with pytest.raises(K.KvselError):
            K.set_sync_wait_us(1000001)
        assert K.set_sync_wait_us(0) == 0
    finally:
        K.set_sync_wait_us(prev)


@pytest.mark.parametrize("kw,status", [
    (dict(cum=None), K.KVSEL_ERR_INVALID),                       # blocks aggregate cum
    (dict(blk_max=None, blk_mean=None), K.KVSEL_ERR_INVALID),
    (dict(block_size=0), K.KVSEL_ERR_INVALID),
    (dict(head_stride=15), K.KVSEL_ERR_INVALID),                 # 1024 / 64 = 16 blocks
    (dict(seq_stride=16 * 8 - 1), K.KVSEL_ERR_INVALID),
    (dict(wsb=0), K.KVSEL_ERR_WORKSPACE),
])
def test_decode_agg_validation(kw, status):
    lib = K.library()
    a = dict(cum=FAKE, blk_max=FAKE, blk_mean=FAKE, block_size=64, head_stride=16, seq_stride=16 * 8,
             wsb=1 << 30)
    a.update(kw)
    st = lib.kvsel_decode_attn_scores_agg(ctypes.byref(_kv()), FAKE, 32, 0.1, FAKE, None, FAKE, 1024,
                                          a["cum"], 1024, 1.0, a["block_size"], a["blk_max"], a["blk_mean"],
                                          a["head_stride"], a["seq_stride"], FAKE, a["wsb"], None)
    assert st == status


def test_quest_validation():
    lib = K.library()
    kv = _kv()          # page 16, max_seq_len 1024: 64 whole pages
    assert lib.kvsel_quest_summarize(None, 0, FAKE, None) == K.KVSEL_ERR_INVALID
    assert lib.kvsel_quest_summarize(ctypes.byref(kv), 0, None, None) == K.KVSEL_ERR_INVALID
    assert lib.kvsel_quest_summarize(ctypes.byref(kv), -1, FAKE, None) == K.KVSEL_ERR_INVALID
    assert lib.kvsel_quest_summarize(ctypes.byref(_kv(head_dim=96)), 0, FAKE, None) == K.KVSEL_ERR_UNSUPPORTED

    def call(kvd=kv, hq=32, summary=FAKE, budget=8, bounds=None, bstride=0, out=FAKE, ostride=8 * 16 + 15,
             ws=FAKE, wsb=1 << 30):
        return lib.kvsel_quest_select(ctypes.byref(kvd), summary, FAKE, hq, budget, bounds, bstride, out,
                                      ostride, FAKE, ws, wsb, None)
    assert call(summary=None) == K.KVSEL_ERR_INVALID
    assert call(out=None) == K.KVSEL_ERR_INVALID
    assert call(budget=-1) == K.KVSEL_ERR_INVALID
    assert call(ostride=8 * 16 + 14) == K.KVSEL_ERR_INVALID     # 8 pages + a partial page
    assert call(budget=100, ostride=1023) == K.KVSEL_ERR_INVALID  # capped at max_seq_len
    assert call(bounds=FAKE, bstride=63) == K.KVSEL_ERR_INVALID
    assert call(hq=24, kvd=_kv(num_kv_heads=4)) == K.KVSEL_ERR_UNSUPPORTED   # G = 6
    assert call(ws=None) == K.KVSEL_ERR_WORKSPACE
    need = lib.kvsel_quest_workspace_bytes(ctypes.byref(kv), 32, 8)
    assert need >= 2 * 32 * 64 * 4              # the bounds rows of every (sequence, head)
    assert call(wsb=need - 1) == K.KVSEL_ERR_WORKSPACE

    def causal(qpos=FAKE, summary=FAKE, ws=FAKE, wsb=1 << 30, ostride=8 * 16 + 15):
        return lib.kvsel_quest_select_causal(ctypes.byref(kv), summary, FAKE, 32, 8, qpos, None, 0, FAKE,
                                             ostride, FAKE, ws, wsb, None)
    assert causal(qpos=None) == K.KVSEL_ERR_INVALID
    assert causal(summary=None) == K.KVSEL_ERR_INVALID
    assert causal(ostride=8 * 16 + 14) == K.KVSEL_ERR_INVALID
    assert causal(ws=None) == K.KVSEL_ERR_WORKSPACE


def test_h2o_validation():
    lib = K.library()

    def call(kvd=None, hq=32, slots=FAKE, out=FAKE, stride=80, sinks=4, window=16, budget=64, ws=FAKE,
             wsb=1 << 30):
        kvd = kvd or _kv()
        return lib.kvsel_h2o_step(ctypes.byref(kvd), FAKE, hq, 0.1, slots, FAKE, FAKE, stride, sinks, window,
                                  budget, None, 1.0, out, None, ws, wsb, None)
    assert call(slots=None) == K.KVSEL_ERR_INVALID
    assert call(out=None) == K.KVSEL_ERR_INVALID
    assert call(kvd=_kv(v_pages=None)) == K.KVSEL_ERR_INVALID
    assert call(budget=-1) == K.KVSEL_ERR_INVALID
    assert call(stride=64) == K.KVSEL_ERR_INVALID                  # no room for the appended token
    assert call(sinks=40, window=40, stride=80) == K.KVSEL_ERR_INVALID
    assert call(hq=96, kvd=_kv(num_kv_heads=8)) == K.KVSEL_ERR_UNSUPPORTED   # G = 12
    assert call(hq=128) == K.KVSEL_ERR_UNSUPPORTED                 # G = 16: lists are shared by a group
    assert call(ws=None) == K.KVSEL_ERR_WORKSPACE
    need = lib.kvsel_h2o_workspace_bytes(ctypes.byref(_kv()), 32, 80, 4, 16, 64)
    assert need >= 2 * 32 * 80 * 4                                 # the logits of every listed slot
    assert call(wsb=need - 1) == K.KVSEL_ERR_WORKSPACE


def test_variant_validation():
    lib = K.library()
    acc = lib.kvsel_accumulate_ex
    assert acc(None, 8, FAKE, 1, 4, 1, 8, 1, 1.0, 0, 0, None, FAKE, 8, None) == K.KVSEL_ERR_INVALID
    assert acc(FAKE, 8, FAKE, 1, 4, 1, 8, 3, 1.0, 0, 0, None, FAKE, 8, None) == K.KVSEL_ERR_INVALID   # mode
    assert acc(FAKE, 8, FAKE, 1, 4, 1, 8, 2, 1.0, 4, 0, None, FAKE, 8, None) == K.KVSEL_ERR_INVALID   # no ring
    assert acc(FAKE, 8, FAKE, 1, 4, 1, 8, 2, 1.0, 0, 0, FAKE, FAKE, 8, None) == K.KVSEL_ERR_INVALID   # window 0
    assert acc(FAKE, 8, FAKE, 1, 4, 1, 8, 2, 1.0, 4, -1, FAKE, FAKE, 8, None) == K.KVSEL_ERR_INVALID  # step < 0
    assert acc(FAKE, 7, FAKE, 1, 4, 1, 8, 1, 1.0, 0, 0, None, FAKE, 8, None) == K.KVSEL_ERR_INVALID   # stride
    blk = lib.kvsel_block_aggregate_ex
    assert blk(FAKE, 64, FAKE, 1, 1, 64, 16, 0, 0.5, None, 4, None) == K.KVSEL_ERR_INVALID
    assert blk(FAKE, 64, FAKE, 1, 1, 64, 16, 3, 0.5, FAKE, 4, None) == K.KVSEL_ERR_INVALID
    assert blk(FAKE, 64, FAKE, 1, 1, 64, 16, 0, 0.5, FAKE, 3, None) == K.KVSEL_ERR_INVALID
    assert blk(FAKE, 1024, FAKE, 1, 1, 1024, 512, 0, 0.5, FAKE, 4, None) == K.KVSEL_ERR_UNSUPPORTED
    thr = lib.kvsel_select_threshold
    assert thr(FAKE, 100, FAKE, 4, 100, 0.5, None, 100, FAKE, None) == K.KVSEL_ERR_INVALID
    assert thr(FAKE, 100, FAKE, 4, 100, 0.5, FAKE, 99, FAKE, None) == K.KVSEL_ERR_INVALID
    assert thr(FAKE, 100, FAKE, 0, 100, 0.5, FAKE, 100, FAKE, None) == K.KVSEL_ERR_INVALID


def test_block_update_validation():
    lib = K.library()
    f = lib.kvsel_block_update
    assert f(None, 8, FAKE, 1, 8, None, 0, 16, 1, 1.0, FAKE, 4, None) == K.KVSEL_ERR_INVALID
    assert f(FAKE, 8, FAKE, 1, 8, None, 0, 0, 1, 1.0, FAKE, 4, None) == K.KVSEL_ERR_INVALID     # block
    assert f(FAKE, 8, FAKE, 0, 8, None, 0, 16, 1, 1.0, FAKE, 4, None) == K.KVSEL_ERR_INVALID     # rows
    assert f(FAKE, 7, FAKE, 1, 8, None, 0, 16, 1, 1.0, FAKE, 4, None) == K.KVSEL_ERR_INVALID     # stride
    assert f(FAKE, 8, FAKE, 1, 8, FAKE, 7, 16, 1, 1.0, FAKE, 4, None) == K.KVSEL_ERR_INVALID     # values
    assert f(FAKE, 8, FAKE, 1, 8, None, 0, 16, 1, 1.0, None, 4, None) == K.KVSEL_ERR_INVALID
    assert f(FAKE, 8, FAKE, 65536, 8, None, 0, 16, 1, 1.0, FAKE, 4, None) == K.KVSEL_ERR_UNSUPPORTED


def test_read_probe_validation():
    lib = K.library()
    f = lib.kvsel_read_probe
    assert f(None, 1024, FAKE, None) == K.KVSEL_ERR_INVALID
    assert f(FAKE, 1024, None, None) == K.KVSEL_ERR_INVALID
    assert f(FAKE + 4, 1024, FAKE, None) == K.KVSEL_ERR_INVALID       # misaligned
    assert f(FAKE, 1000, FAKE, None) == K.KVSEL_ERR_INVALID           # not a multiple of 16


def test_union_validation():
    lib = K.library()
    u = lib.kvsel_union_keep
    assert u(None, 8, FAKE, 1, 4, 2, 100, FAKE, 16, FAKE, None) == K.KVSEL_ERR_INVALID
    assert u(FAKE, 8, FAKE, 1, 6, 4, 100, FAKE, 16, FAKE, None) == K.KVSEL_ERR_INVALID    # 6 % 4
    assert u(FAKE, 8, FAKE, 1, 4, 2, 100, FAKE, 15, FAKE, None) == K.KVSEL_ERR_INVALID    # 2 x 8 = 16 slots
    assert u(FAKE, 8, FAKE, 1, 4, 2, (1 << 20) + 1, FAKE, 16, FAKE, None) == K.KVSEL_ERR_UNSUPPORTED


def test_indexer_fp8_validation():
    lib = K.library()
    f = lib.kvsel_indexer_scores_fp8
    kv8 = _kv(dtype=K.KVSEL_FP8_E4M3, v_pages=None)
    assert f(ctypes.byref(_kv()), FAKE, 32, 1.0, FAKE, 1024, None) == K.KVSEL_ERR_INVALID      # bf16 pages
    assert f(ctypes.byref(kv8), None, 32, 1.0, FAKE, 1024, None) == K.KVSEL_ERR_INVALID
    assert f(ctypes.byref(kv8), FAKE, 32, 1.0, FAKE, 1000, None) == K.KVSEL_ERR_INVALID         # stride
    assert f(ctypes.byref(kv8), FAKE + 4, 32, 1.0, FAKE, 1024, None) == K.KVSEL_ERR_INVALID     # unaligned q
    assert f(ctypes.byref(_kv(dtype=K.KVSEL_FP8_E4M3, head_dim=96)), FAKE, 32, 1.0, FAKE, 1024,
             None) == K.KVSEL_ERR_UNSUPPORTED
    # the other calls refuse FP8 pages
    assert _decode(_kv(dtype=K.KVSEL_FP8_E4M3)) == K.KVSEL_ERR_UNSUPPORTED


def test_indexer_topk_validation():
    """bf16 and FP8 E4M3 pages are taken (the FP8 q and pages 16-byte
    aligned), f32 pages are not; everything else fails before any HIP call."""
    lib = K.library()
    f, wsq = lib.kvsel_indexer_topk, lib.kvsel_indexer_topk_workspace_bytes
    kv16 = _kv(num_kv_heads=1, head_dim=64, v_pages=None)
    kv8 = _kv(num_kv_heads=1, head_dim=64, v_pages=None, dtype=K.KVSEL_FP8_E4M3)

    def call(kvd, q=FAKE, topk=256, keep=FAKE, kstride=256, ws=FAKE, wsb=1 << 30):
        return f(ctypes.byref(kvd), q, 32, 1.0, topk, keep, kstride, FAKE, ws, wsb, None)

    assert wsq(ctypes.byref(kv16), 32, 256) > 0 and wsq(ctypes.byref(kv8), 32, 256) > 0
    assert wsq(ctypes.byref(_kv(num_kv_heads=1, head_dim=64, dtype=K.KVSEL_F32)), 32, 256) == 0
    for kvd in (kv16, kv8):
        assert call(kvd, q=None) == K.KVSEL_ERR_INVALID
        assert call(kvd, topk=0) == K.KVSEL_ERR_INVALID
        assert call(kvd, kstride=100) == K.KVSEL_ERR_INVALID
        assert call(kvd, wsb=16) == K.KVSEL_ERR_WORKSPACE
    assert call(kv8, q=FAKE + 8) == K.KVSEL_ERR_INVALID                                    # unaligned FP8 q
    assert call(_kv(num_kv_heads=1, head_dim=64, v_pages=None, dtype=K.KVSEL_FP8_E4M3, k_pages=FAKE + 4)) == \
        K.KVSEL_ERR_INVALID                                                                  # unaligned FP8 pages
    assert call(_kv(num_kv_heads=1, head_dim=64, v_pages=None, dtype=K.KVSEL_F32)) == K.KVSEL_ERR_UNSUPPORTED
    assert call(_kv(num_kv_heads=1, head_dim=96, v_pages=None, dtype=K.KVSEL_FP8_E4M3)) == K.KVSEL_ERR_UNSUPPORTED


def test_noalloc_decode_rejects_before_hip():
    """The allocation-free decode validates like the workspace variant and
    rejects a call whose workspace would exceed the static scratch, all
    before any HIP call.  The limit the binding states is the header's."""
    import os
    lib = K.library()
    hdr = open(os.path.join(os.path.dirname(__file__), "..", HEADER)).read()
    m = re.search(r"#define KVSEL_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == K.NOALLOC_SCRATCH_BYTES

    def call(kv, hq=32, probs=FAKE, cum=None, q=FAKE, out=FAKE):
        return lib.kvsel_decode_attn_scores_noalloc(ctypes.byref(kv), q, hq, 0.1, out, None, probs,
                                                    kv.max_seq_len, 0, cum, kv.max_seq_len, 1.0, None)
    assert call(_kv(), q=None) == K.KVSEL_ERR_INVALID
    assert call(_kv(v_pages=None)) == K.KVSEL_ERR_INVALID
    assert call(_kv(), hq=30) == K.KVSEL_ERR_INVALID
    assert call(_kv(head_dim=96)) == K.KVSEL_ERR_UNSUPPORTED
    # 8 x 64 heads x 1M keys with cum and no probs: a 2 GiB logits scratch
    big = _kv(num_seqs=8, max_seq_len=1 << 20, max_pages_per_seq=1 << 16)
    assert call(big, hq=64, probs=None, cum=FAKE) == K.KVSEL_ERR_WORKSPACE
    assert b"static scratch" in lib.kvsel_last_error()
    # the workspace the same call would need, for comparison
    assert lib.kvsel_decode_workspace_bytes(ctypes.byref(big), 64, 0) > K.NOALLOC_SCRATCH_BYTES
