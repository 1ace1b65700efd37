"""Pins of the oracle's top-k (O2): brute force with Python's own sort, set
invariants and the degenerate rows.  The k best are taken in the order (score
desc, index asc), the order of packed keys with the score above an inverted index
("Latent Sparse Attention" article, section "What the kernels do about the
top-p"), and listed in ascending index order (the same section notes the list is
never sorted because attention does not depend on its order)."""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("seed", range(5))
def test_brute_force_small_rows(seed):
    rng = np.random.default_rng(seed)
    R, S = 7, 37
    # few distinct values -> many ties
    scores = rng.integers(-3, 4, (R, S)).astype(np.float64) * 0.5
    nv = rng.integers(0, S + 1, R).astype(np.int32)
    for k in (1, 5, 16, 37, 45):
        idx, val = oracle.topk(scores, k, nv)
        for r in range(R):
            ref = sorted(sorted(range(int(nv[r])), key=lambda i: (-scores[r, i], i))[:k])
            n = len(ref)
            assert list(idx[r, :n]) == ref
            assert np.all(idx[r, n:] == -1) and np.all(np.isneginf(val[r, n:]))
            assert np.array_equal(val[r, :n], scores[r, ref])


def test_set_invariants():
    rng = np.random.default_rng(9)
    R, S, k = 5, 3000, 256
    scores = rng.standard_normal((R, S))
    idx, val = oracle.topk(scores, k)
    for r in range(R):
        sel = idx[r]
        assert len(set(sel.tolist())) == k and sel.min() >= 0 and sel.max() < S
        rest = np.setdiff1d(np.arange(S), sel)
        assert scores[r, sel].min() >= scores[r, rest].max()
        assert np.all(np.diff(sel) > 0)
        assert np.array_equal(val[r], scores[r, sel])


def test_all_equal_row_and_signed_zero():
    s = np.zeros((2, 10))
    s[1, ::2] = -0.0
    idx, _ = oracle.topk(s, 4)
    assert idx.tolist() == [[0, 1, 2, 3], [0, 1, 2, 3]]


def test_negative_scores_and_padding():
    s = np.array([[-5.0, -1.0, -3.0, -np.inf, 2.0]])
    idx, val = oracle.topk(s, 7, nv=np.array([4], np.int32))
    assert idx.tolist() == [[0, 1, 2, 3, -1, -1, -1]]
    assert val[0, 3] == -np.inf and np.isneginf(val[0, 4:]).all()
