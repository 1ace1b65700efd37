"""Pins of the oracle's sparse attention (O4): exact attention over only the
selected latent rows ("Long context" lecture, section "The Architectural
Answer", paragraph "Stage 2, sparse main attention"); values are the first dv
elements of each row."""
import math

import numpy as np
from scipy.special import logsumexp

import oracle
import synth


def _bf(u16):
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _problem(seed, B=2, Hq=4, S=50, k=12, dqk=24, dv=16):
    rng = np.random.default_rng(seed)
    q = synth.normal_bf16(seed, 1, (B, Hq, dqk))
    kv = synth.normal_bf16(seed, 2, (B, S, dqk))
    idx = np.stack([rng.choice(S, k, replace=False) for _ in range(B)]).astype(np.int32)
    return q, kv, idx, dv


def test_matches_dense_softmax_on_gathered_rows():
    q, kv, idx, dv = _problem(0)
    tau = 1 / math.sqrt(192)
    out, lse = oracle.sparse_attn(q, kv, idx, dv, tau)
    for b in range(q.shape[0]):
        K = _bf(kv[b, idx[b]])
        logits = tau * (_bf(q[b]) @ K.T)
        p = np.exp(logits - logits.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        np.testing.assert_allclose(out[b], p @ K[:, :dv], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[b], logsumexp(logits, axis=1), rtol=1e-13)


def test_single_row_and_zero_query():
    q, kv, idx, dv = _problem(1)
    out, lse = oracle.sparse_attn(q, kv, idx[:, :1], dv, 0.3)
    for b in range(q.shape[0]):
        assert np.array_equal(out[b], np.broadcast_to(_bf(kv[b, idx[b, 0], :dv]), out[b].shape))
    z = np.zeros_like(q)
    out, lse = oracle.sparse_attn(z, kv, idx, dv, 0.3)
    for b in range(q.shape[0]):
        np.testing.assert_allclose(out[b], np.broadcast_to(_bf(kv[b, idx[b], :dv]).mean(0), out[b].shape), rtol=1e-13)
        np.testing.assert_allclose(lse[b], math.log(idx.shape[1]), rtol=1e-14)


def test_permutation_and_skipped_entries():
    q, kv, idx, dv = _problem(2)
    out, lse = oracle.sparse_attn(q, kv, idx, dv, 0.2)
    perm = np.random.default_rng(0).permutation(idx.shape[1])
    o2, l2 = oracle.sparse_attn(q, kv, idx[:, perm], dv, 0.2)
    np.testing.assert_allclose(o2, out, rtol=1e-12, atol=1e-14)
    padded = np.concatenate([idx, -np.ones((idx.shape[0], 5), np.int32)], axis=1)
    o3, l3 = oracle.sparse_attn(q, kv, padded, dv, 0.2)
    np.testing.assert_allclose(o3, out, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(l3, lse, rtol=1e-15)
    o4, l4 = oracle.sparse_attn(q, kv, -np.ones_like(idx), dv, 0.2)
    assert (o4 == 0).all() and np.isneginf(l4).all()


def test_pre_gathered_rows_match_dense_softmax():
    # the entry point over rows already gathered (row i of b is kv[b, idx[b, i]]),
    # with skipped entries (-1) given as zero rows, against numpy's dense softmax
    # over the kept rows only
    q, kv, idx, dv = _problem(3, k=10)
    idx = idx.copy()
    idx[0, [2, 7]] = -1
    idx[1, 0] = -1
    rows = np.zeros((q.shape[0], idx.shape[1], q.shape[2]), np.uint16)
    for b in range(q.shape[0]):
        for i, s in enumerate(idx[b]):
            if s >= 0:
                rows[b, i] = kv[b, s]
    tau = 0.25
    out, lse = oracle.sparse_attn_rows(q, rows, idx, dv, tau)
    for b in range(q.shape[0]):
        keep = idx[b] >= 0
        K = _bf(rows[b][keep])
        logits = tau * (_bf(q[b]) @ K.T)
        p = np.exp(logits - logits.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        np.testing.assert_allclose(out[b], p @ K[:, :dv], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[b], logsumexp(logits, axis=1), rtol=1e-13)
