"""Pins of the oracle's product-quantised two-stage search (O7), LeanSparse podcast
transcript cues 07:12-08:00: each 128-d key split into 32 four-dimension pieces,
each piece a one-byte index into a 256-entry codebook; the coarse pass over the
codes keeps 2,048 candidates and an exact rerank of their original keys picks
512.  The coarse score is the asymmetric one (the query is not quantised by the
codebook): the lookup-table sum over pieces equals the dot with the decoded key,
which the pins check with independent numpy arithmetic.  Recall values on
synthetic keys are parity unpinned (the pages' figures are for real traces)."""
import numpy as np
import pytest

import oracle
import synth
from synth import workloads


def _bf(u16):
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _small(seed=0, B=3, S=900, H=8):
    sp = workloads.spec("pq_search", B=B, S=S, H=H, seed=0x5EED0F00 + seed, pq_train_stride=1, pq_iters=4)
    return sp, workloads.pq_inputs(sp)


def test_query_codes_match_numpy():
    sp, x = _small(0)
    q8, W = oracle.pq_query(x["q"], x["w"], x["sigma"])
    qf = _bf(x["q"])
    qs = np.abs(qf).max(-1) / 127
    t = qf / qs[..., None]
    ok = np.abs(np.abs(t - np.trunc(t)) - 0.5) > 1e-9
    assert np.array_equal(np.clip(np.rint(t), -127, 127)[ok], q8.astype(np.float64)[ok])
    np.testing.assert_allclose(W, x["w"].astype(np.float64) * qs * x["sigma"], rtol=1e-15)


def test_lookup_table_sum_equals_decoded_dot():
    sp, x = _small(1)
    B, S, H, d = sp["B"], sp["S"], sp["H"], sp["d"]
    q8, W = oracle.pq_query(x["q"], x["w"], x["sigma"])
    res = oracle.pq_search(x["q"], x["w"], x["cb"], x["sigma"], x["codes"], x["k_full"], 64, 16, want_s1=True)
    cb = x["cb"].astype(np.int64)
    codes = x["codes"].astype(np.int64)
    q = q8.astype(np.int64).reshape(B, H, d // 4, 4)
    # asymmetric lookup tables: L[b, h, j, c] = q8_h[piece j] . entry c of piece j
    lut = np.einsum("bhji,jci->bhjc", q, cb)
    D_lut = np.zeros((B, H, S), np.int64)
    for j in range(d // 4):
        D_lut += np.take_along_axis(lut[:, :, j, :], codes[:, None, :, j].repeat(H, axis=1), axis=2)
    # brute force: decode every key, plain integer dot
    dec = cb[np.arange(d // 4)[None, None, :], codes].reshape(B, S, d)
    D_dec = np.einsum("bhd,bsd->bhs", q8.astype(np.int64), dec)
    assert np.array_equal(D_lut, D_dec)
    ref = (W[..., None] * np.maximum(D_dec, 0)).sum(axis=1)
    np.testing.assert_allclose(res["s1"], ref, rtol=1e-13)
    sl, _ = oracle.topk(res["s1"], 64)
    assert np.array_equal(sl, res["shortlist"])


def test_reconstructed_keys_score_exactly():
    # keys that are codebook reconstructions (sigma a power of two, so exact in
    # bf16) and integer queries whose largest magnitude is 127 (so their int8 codes
    # are themselves, scale 1): the coarse score is the exact score of O1, bit for bit
    rng = np.random.default_rng(5)
    B, S, H, d = 2, 300, 6, 128
    cb = rng.integers(-127, 128, (32, 256, 4)).astype(np.int8)
    sigma = 2.0 ** -5
    codes = rng.integers(0, 256, (B, S, 32)).astype(np.uint8)
    keys = sigma * cb[np.arange(32)[None, None, :], codes].reshape(B, S, d).astype(np.float64)
    k_bf = np.array([synth.bf16_rne(v) for v in keys.ravel()], np.uint16).reshape(B, S, d)
    assert np.array_equal(_bf(k_bf), keys)
    qi = rng.integers(-127, 128, (B, H, d)).astype(np.float64)
    qi[:, :, 0] = 127
    q = np.array([synth.bf16_rne(v) for v in qi.ravel()], np.uint16).reshape(B, H, d)
    w = rng.random((B, H)).astype(np.float32)
    res = oracle.pq_search(q, w, cb, sigma, codes, k_bf, 32, 8, want_s1=True)
    exact = oracle.indexer_score(q.reshape(B, 1, H, d), oracle.BF16, w.reshape(B, 1, H), k_bf, oracle.BF16)
    assert np.array_equal(res["s1"], exact)


def test_full_shortlist_equals_exact_topk():
    sp, x = _small(2, S=400)
    B, S, H, d = sp["B"], sp["S"], sp["H"], sp["d"]
    res = oracle.pq_search(x["q"], x["w"], x["cb"], x["sigma"], x["codes"], x["k_full"], m=S, k=40)
    exact = oracle.indexer_score(x["q"].reshape(B, 1, H, d), oracle.BF16, x["w"].reshape(B, 1, H),
                                 x["k_full"], oracle.BF16)
    idx, val = oracle.topk(exact, 40)
    assert np.array_equal(res["idx"], idx) and np.array_equal(res["val"], val)


def test_recall_identity_monotone_and_visible_counts():
    sp, x = _small(3, S=2000)
    B, S, H, d, k = sp["B"], sp["S"], sp["H"], sp["d"], 32
    exact = oracle.indexer_score(x["q"].reshape(B, 1, H, d), oracle.BF16, x["w"].reshape(B, 1, H),
                                 x["k_full"], oracle.BF16)
    true_idx, _ = oracle.topk(exact, k)
    prev = None
    for m in (32, 128, 512, 2000):
        res = oracle.pq_search(x["q"], x["w"], x["cb"], x["sigma"], x["codes"], x["k_full"], m=m, k=k)
        rec = []
        for b in range(B):
            t = set(true_idx[b].tolist())
            fin, sl = set(res["idx"][b].tolist()), set(res["shortlist"][b].tolist())
            assert fin & t == sl & t
            rec.append(len(fin & t) / k)
        r = float(np.mean(rec))
        assert prev is None or r >= prev
        prev = r
    assert prev == 1.0
    nv = np.array([5, 2000, 700], np.int32)
    res = oracle.pq_search(x["q"], x["w"], x["cb"], x["sigma"], x["codes"], x["k_full"], m=64, k=16, nv=nv)
    assert (res["shortlist"][0, 5:] == -1).all() and set(res["idx"][0, :5].tolist()) == set(range(5))
    assert res["idx"][2].max() < 700
