"""Pins of the oracle's two-stage compact search (O3), LeanSparse podcast
transcript cues 07:12-08:00: a coarse pass over compact keys keeps a shortlist,
the shortlisted original keys are rescored exactly and the best k kept.
Recall values on synthetic keys are parity unpinned (the pages give none for
this encoding); what is pinned is the arithmetic and the reductions below."""
import math

import numpy as np

import oracle
import synth
from synth import workloads


def _small(seed=0, B=3, S=700, H=8):
    sp = workloads.spec("compact_search", B=B, S=S, H=H, seed=seed)
    return sp, workloads.compact_inputs(sp)


def _bf(u16):
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_compact_key_encoding_matches_numpy():
    sp, x = _small()
    y = _bf(x["k_full"]) @ x["P"].astype(np.float64).T  # [B, S, dc]
    amax = np.abs(y).max(axis=-1)
    cs = (amax / 127).astype(np.float32)
    assert np.array_equal(cs, x["cs"])
    t = y / cs[..., None].astype(np.float64)
    near_half = np.abs(np.abs(t - np.trunc(t)) - 0.5) < 1e-9
    ref = np.clip(np.rint(t), -127, 127)
    assert np.array_equal(ref[~near_half], x["c"].astype(np.float64)[~near_half])


def test_query_encoding_and_stage1_scores():
    sp, x = _small(seed=1)
    q8, qs, W = oracle.compact_query(x["q"], x["w"], x["P"])
    y = _bf(x["q"]) @ x["P"].astype(np.float64).T  # [B, H, dc]
    np.testing.assert_allclose(qs, np.abs(y).max(-1) / 127, rtol=1e-14)
    t = y / qs[..., None]
    ok = np.abs(np.abs(t - np.trunc(t)) - 0.5) > 1e-9
    assert np.array_equal(np.clip(np.rint(t), -127, 127)[ok], q8.astype(np.float64)[ok])
    np.testing.assert_allclose(W, x["w"].astype(np.float64) * qs, rtol=1e-15)
    res = oracle.compact_search(x["q"], x["w"], x["P"], x["c"], x["cs"], x["k_full"], m=64, k=16, want_s1=True)
    D = np.einsum("bhi,bsi->bhs", q8.astype(np.int64), x["c"].astype(np.int64))  # exact integers
    ref = x["cs"].astype(np.float64) * (W[..., None] * np.maximum(D, 0)).sum(axis=1)
    np.testing.assert_allclose(res["s1"], ref, rtol=1e-13)
    # the shortlist is the top-m set of s1 (ties to the smaller index)
    sl, _ = oracle.topk(res["s1"], 64)
    assert np.array_equal(sl, res["shortlist"])


def test_full_shortlist_equals_exact_topk():
    sp, x = _small(seed=2, S=300)
    B, S, H, d = sp["B"], sp["S"], sp["H"], sp["d"]
    res = oracle.compact_search(x["q"], x["w"], x["P"], x["c"], x["cs"], x["k_full"], m=S, k=40)
    exact = oracle.indexer_score(x["q"].reshape(B, 1, H, d), oracle.BF16, x["w"].reshape(B, 1, H),
                                 x["k_full"], oracle.BF16)
    idx, val = oracle.topk(exact, 40)
    assert np.array_equal(res["idx"], idx) and np.array_equal(res["val"], val)


def test_recall_identity_and_monotone_in_m():
    sp, x = _small(seed=3, S=2000)
    B, S, H, d, k = sp["B"], sp["S"], sp["H"], sp["d"], 32
    exact = oracle.indexer_score(x["q"].reshape(B, 1, H, d), oracle.BF16, x["w"].reshape(B, 1, H),
                                 x["k_full"], oracle.BF16)
    true_idx, _ = oracle.topk(exact, k)
    prev = None
    for m in (32, 64, 128, 512, 2000):
        res = oracle.compact_search(x["q"], x["w"], x["P"], x["c"], x["cs"], x["k_full"], m=m, k=k)
        rec = []
        for b in range(B):
            t = set(true_idx[b].tolist())
            fin = set(res["idx"][b].tolist())
            sl = set(res["shortlist"][b].tolist())
            # the exact rerank keeps every true top-k key that made the shortlist
            assert fin & t == sl & t
            rec.append(len(fin & t) / k)
        r = float(np.mean(rec))
        if prev is not None:
            assert r >= prev
        prev = r
    assert prev == 1.0


def test_nv_below_shortlist_pads():
    sp, x = _small(seed=4, S=200)
    nv = np.array([5, 200, 150], np.int32)
    res = oracle.compact_search(x["q"], x["w"], x["P"], x["c"], x["cs"], x["k_full"], m=64, k=16, nv=nv)
    assert (res["shortlist"][0, 5:] == -1).all() and (res["idx"][0, 5:] == -1).all()
    assert set(res["idx"][0, :5].tolist()) == set(range(5))
    assert res["idx"][2].max() < 150
