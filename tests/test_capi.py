"""The C ABI library loads, exports every entry point include/li.h declares, and
rejects bad arguments on the host before launching anything (no GPU needed)."""
import ctypes
import os
import re

import pytest

import lightning_indexer_top_amd as li

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "li.h")

A = ctypes.c_void_p(0x10000)        # aligned fake device pointer (never dereferenced)
A2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10004)      # misaligned
NUL = None


def declared(hdr=HDR):
    text = open(hdr).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(li_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = li.lib()
    names = declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert li.lib().li_version().startswith(b"lightning-indexer")


def test_probe_library_exports_its_header():
    from lightning_indexer_top_amd import build as b
    L = ctypes.CDLL(b.PROBE_LIB)
    names = declared(os.path.join(ROOT, "include", "li_probe.h"))
    assert len(names) == 5
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    L = li.lib()
    for s in range(7):
        assert L.li_status_string(s)
    assert L.li_status_string(99) == b"unknown status"


def _score(**kw):
    a = dict(q=A, qt=li.LI_BF16, w=A, k=A, kt=li.LI_FP8_E4M3, ks=A, nv=NUL, B=1, T=1, S=100, H=64, d=128, out=A)
    a.update(kw)
    return li.lib().li_indexer_score(a["q"], a["qt"], a["w"], a["k"], a["kt"], a["ks"], a["nv"], a["B"], a["T"],
                                     a["S"], a["H"], a["d"], a["out"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=NUL), 1), (dict(w=NUL), 1), (dict(k=NUL), 1), (dict(out=NUL), 1), (dict(ks=NUL), 1),
    (dict(d=64), 2), (dict(H=0), 2), (dict(H=129), 2), (dict(S=0), 2), (dict(B=0), 2), (dict(T=-1), 2),
    (dict(qt=li.LI_FP8_E4M3), 3), (dict(kt=li.LI_I8), 3), (dict(kt=li.LI_BF16), 3),
    (dict(q=MIS), 4), (dict(out=MIS), 4), (dict(nv=MIS), 4),
    (dict(B=1 << 16, T=1 << 14, S=1 << 12), 2),
])
def test_indexer_score_rejects(kw, status):
    assert _score(**kw) == status
    assert li.lib().li_last_error()


def test_topk_rejects():
    L = li.lib()
    assert L.li_topk_select(NUL, NUL, 4, 100, 8, A, A, NUL, 0, None) == 1
    assert L.li_topk_select(A, NUL, 4, 100, 0, A, A, NUL, 0, None) == 2
    assert L.li_topk_select(A, NUL, 4, 100, 2049, A, A, NUL, 0, None) == 2
    assert L.li_topk_select(A, NUL, 0, 100, 8, A, A, NUL, 0, None) == 2
    assert L.li_topk_select(A, NUL, 4, 100, 8, MIS, A, NUL, 0, None) == 4


def test_indexer_topk_rejects():
    L = li.lib()
    args = [A, li.LI_BF16, A, A, li.LI_BF16, NUL, NUL, 1, 16, 1000, 64, 128]
    assert L.li_indexer_topk(*args, 0, A, A, A, 1 << 30, None) == 2
    assert L.li_indexer_topk(*args, 2049, A, A, A, 1 << 30, None) == 2
    assert L.li_indexer_topk(*args, 16, NUL, A, A, 1 << 30, None) == 1
    # decode-shaped rows (fp8 keys, one row per sequence) need a workspace
    fargs = [A, li.LI_BF16, A, A, li.LI_FP8_E4M3, A, NUL, 4, 1, 100000, 64, 128]
    need = L.li_indexer_topk_workspace_bytes(li.LI_BF16, li.LI_FP8_E4M3, 4, 1, 100000, 64, 512)
    assert need > 4 * 100000 * 4
    assert L.li_indexer_topk(*fargs, 512, A, A, NUL, 0, None) == 5
    assert L.li_indexer_topk(*fargs, 512, A, A, A, need - 1, None) == 5


def test_indexer_topk_workspace_follows_the_path():
    L = li.lib()
    ws = L.li_indexer_topk_workspace_bytes
    # the fused many-row kernel (bf16 queries and keys, T >= 16, k <= 512) needs
    # none: the prefill chunk (4096 rows over 131072 keys) asks for 0 bytes
    assert ws(li.LI_BF16, li.LI_BF16, 1, 4096, 131072, 64, 512) == 0
    assert ws(li.LI_BF16, li.LI_BF16, 1, 16, 1000, 64, 16) == 0
    # fp8 keys take the same tiled kernel (the fp8 tiles widened to bf16 in LDS)
    assert ws(li.LI_BF16, li.LI_FP8_E4M3, 1, 16, 1000, 64, 16) == 0
    # past the fused kernel's k (512) the call scores then selects: the score matrix
    # plus the top-k's own workspace
    n = ws(li.LI_BF16, li.LI_FP8_E4M3, 1, 16, 1000, 64, 600)
    assert n >= 16 * 1000 * 4 + L.li_topk_workspace_bytes(16, 1000, 600)
    # decode rows: the scores, then the top-k's thresholds, counts and candidate lists
    assert ws(li.LI_BF16, li.LI_FP8_E4M3, 16, 1, 131072, 64, 512) == \
        16 * 131072 * 4 + L.li_topk_workspace_bytes(16, 131072, 512)
    assert L.li_topk_workspace_bytes(16, 131072, 512) >= 16 * 131072 * 4 * 2
    assert ws(li.LI_BF16, li.LI_BF16, 0, 16, 1000, 64, 16) == 0


def test_compact_rejects():
    L = li.lib()
    need = L.li_compact_workspace_bytes(2, 1000, 64, 256, 64)
    assert need > 0

    def call(**kw):
        a = dict(q=A, w=A, P=A, ck=A, cks=A, kf=A, nv=NUL, B=2, S=1000, H=64, d=128, dc=32, m=256, k=64, sl=A,
                 idx=A, val=A, ws=A2, nb=need)
        a.update(kw)
        return L.li_compact_search_rerank(a["q"], a["w"], a["P"], a["ck"], a["cks"], a["kf"], a["nv"], a["B"],
                                          a["S"], a["H"], a["d"], a["dc"], a["m"], a["k"], a["sl"], a["idx"],
                                          a["val"], a["ws"], a["nb"], None)
    assert call(q=NUL) == 1 and call(kf=NUL) == 1 and call(idx=NUL) == 1
    assert call(dc=16) == 2 and call(d=64) == 2 and call(m=32) == 2 and call(m=4096, k=64) == 2
    assert call(k=0) == 2 and call(H=200) == 2
    assert call(ws=NUL) == 5 and call(nb=need - 1) == 5
    assert call(ck=MIS) == 4


def test_sparse_attn_rejects():
    L = li.lib()

    def call(**kw):
        a = dict(q=A, kv=A, idx=A, B=2, Hq=128, S=1000, k=64, dqk=576, dv=512, sc=0.07, out=A, lse=A)
        a.update(kw)
        return L.li_sparse_attn_gather(a["q"], a["kv"], a["idx"], a["B"], a["Hq"], a["S"], a["k"], a["dqk"],
                                       a["dv"], a["sc"], a["out"], a["lse"], NUL, 0, None)
    assert call(q=NUL) == 1 and call(idx=NUL) == 1 and call(out=NUL) == 1
    assert call(Hq=48) == 2 and call(Hq=256) == 2 and call(dqk=512) == 2 and call(dv=576) == 2
    assert call(k=0) == 2 and call(k=4096) == 2
    assert call(lse=MIS) == 4


def test_topk_noalloc_rejects():
    # validation runs before anything touches the device: fake pointers are safe
    L = li.lib()
    assert L.li_topk_select_noalloc(NUL, NUL, 4, 100, 8, A, A, None) == 1
    assert L.li_topk_select_noalloc(A, NUL, 4, 100, 0, A, A, None) == 2
    assert L.li_topk_select_noalloc(A, NUL, 4, 100, 2049, A, A, None) == 2
    assert L.li_topk_select_noalloc(A, NUL, 0, 100, 8, A, A, None) == 2
    assert L.li_topk_select_noalloc(A, NUL, 4, 100, 8, MIS, A, None) == 4
    # a shape whose selection needs more than the static scratch
    assert L.li_topk_workspace_bytes(64, 262144, 512) > 34078720
    assert L.li_topk_select_noalloc(A, NUL, 64, 262144, 512, A, A, None) == 5
    assert b"static scratch" in L.li_last_error()
    # the largest decode shape it takes
    assert L.li_topk_workspace_bytes(16, 262144, 512) <= 34078720
    assert L.li_topk_workspace_bytes(159, 26379, 512) <= 34078720


def test_pooled_rejects():
    L = li.lib()
    assert L.li_pool_keys(NUL, li.LI_BF16, 2, 100, 128, 4, A, A, None) == 1
    assert L.li_pool_keys(A, li.LI_FP8_E4M3, 2, 100, 128, 4, A, A, None) == 3
    assert L.li_pool_keys(A, li.LI_BF16, 2, 100, 64, 4, A, A, None) == 2
    assert L.li_pool_keys(A, li.LI_BF16, 2, 100, 128, 3, A, A, None) == 2
    assert L.li_pool_keys(A, li.LI_BF16, 2, 100, 128, 4, MIS, A, None) == 4
    assert L.li_pool_keys(NUL, li.LI_BF16, 2, 3, 128, 4, NUL, NUL, None) == 0  # no complete block
    need = L.li_pooled_indexer_topk_workspace_bytes(16, 1, 131072, 32, 512)
    assert need > 16 * 131072 * 4

    def call(**kw):
        a = dict(q=A, qt=li.LI_BF16, w=A, c=A, s=A, nv=NUL, B=16, T=1, Sp=131072, H=32, d=128, pool=4, k=512,
                 idx=A, val=A, ws=A2, nb=need)
        a.update(kw)
        return L.li_pooled_indexer_topk(a["q"], a["qt"], a["w"], a["c"], a["s"], a["nv"], a["B"], a["T"], a["Sp"],
                                        a["H"], a["d"], a["pool"], a["k"], a["idx"], a["val"], a["ws"], a["nb"],
                                        None)
    assert call(q=NUL) == 1 and call(s=NUL) == 1 and call(idx=NUL) == 1
    assert call(qt=li.LI_F32) == 3
    assert call(pool=5) == 2 and call(k=0) == 2 and call(k=4096) == 2 and call(H=0) == 2
    assert call(Sp=1 << 29, pool=8) == 2
    assert call(ws=NUL) == 5 and call(nb=need - 1) == 5
    assert call(idx=MIS) == 4


def test_paged_rejects():
    L = li.lib()

    def score(**kw):
        a = dict(q=A, qt=li.LI_BF16, w=A, k=A, s=A, pt=A, ps=64, mp=2048, npg=40000, nv=NUL, B=16, T=1, S=131072,
                 H=64, d=128, out=A)
        a.update(kw)
        return L.li_indexer_score_paged(a["q"], a["qt"], a["w"], a["k"], a["s"], a["pt"], a["ps"], a["mp"],
                                        a["npg"], a["nv"], a["B"], a["T"], a["S"], a["H"], a["d"], a["out"], None)
    assert score(pt=NUL) == 1 and score(s=NUL) == 1 and score(out=NUL) == 1
    assert score(qt=li.LI_F32) == 3
    assert score(ps=32) == 2 and score(mp=2047) == 2 and score(npg=0) == 2 and score(npg=1 << 25) == 2
    assert score(pt=MIS) == 4
    need = L.li_indexer_topk_paged_workspace_bytes(16, 1, 131072, 64, 512)
    assert need >= L.li_indexer_topk_workspace_bytes(li.LI_BF16, li.LI_FP8_E4M3, 16, 1, 131072, 64, 512)

    def topk(**kw):
        a = dict(pt=A, mp=2048, k=512, ws=A2, nb=need)
        a.update(kw)
        return L.li_indexer_topk_paged(A, li.LI_BF16, A, A, A, a["pt"], 64, a["mp"], 40000, NUL, 16, 1, 131072, 64,
                                       128, a["k"], A, A, a["ws"], a["nb"], None)
    assert topk(pt=NUL) == 1 and topk(mp=100) == 2 and topk(k=0) == 2 and topk(nb=need - 1) == 5
    assert topk(ws=NUL) == 5

    def attn(**kw):
        a = dict(q=A, kv=A, st=A, ms=1000, ns=5000, idx=A, B=2, Hq=128, S=1000, k=64, out=A)
        a.update(kw)
        return L.li_sparse_attn_gather_paged(a["q"], a["kv"], a["st"], a["ms"], a["ns"], a["idx"], a["B"], a["Hq"],
                                             a["S"], a["k"], 576, 512, 0.07, a["out"], NUL, None)
    assert attn(st=NUL) == 1 and attn(kv=NUL) == 1
    assert attn(ms=999) == 2 and attn(ns=0) == 2 and attn(Hq=40) == 2 and attn(k=0) == 2
    assert attn(st=MIS) == 4


def test_pq_rejects():
    L = li.lib()
    need = L.li_pq_workspace_bytes(2, 1000, 64, 256, 64)
    assert need > 0

    def call(**kw):
        a = dict(q=A, w=A, cb=A, sg=0.03, c=A, kf=A, nv=NUL, B=2, S=1000, H=64, d=128, m=256, k=64, sl=A, idx=A,
                 val=A, ws=A2, nb=need)
        a.update(kw)
        return L.li_pq_search_rerank(a["q"], a["w"], a["cb"], a["sg"], a["c"], a["kf"], a["nv"], a["B"], a["S"],
                                     a["H"], a["d"], a["m"], a["k"], a["sl"], a["idx"], a["val"], a["ws"], a["nb"],
                                     None)
    assert call(q=NUL) == 1 and call(cb=NUL) == 1 and call(c=NUL) == 1 and call(idx=NUL) == 1
    assert call(d=64) == 2 and call(m=32) == 2 and call(m=4096, k=64) == 2 and call(k=0) == 2 and call(H=200) == 2
    assert call(sg=0.0) == 2 and call(sg=-1.0) == 2 and call(sg=float("inf")) == 2
    assert call(ws=NUL) == 5 and call(nb=need - 1) == 5
    assert call(c=MIS) == 4
