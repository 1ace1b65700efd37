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


def declared():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(li_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = li.lib()
    names = declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert li.lib().li_version().startswith(b"lightning-indexer")


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
    need = L.li_indexer_topk_workspace_bytes(1, 16, 1000, 64, 16)
    if need:
        assert L.li_indexer_topk(*args, 16, A, A, NUL, 0, None) == 5
        assert L.li_indexer_topk(*args, 16, A, A, A, need - 1, None) == 5


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
