"""GPU parity of li_topk_select: on the same fp32 scores the GPU selection must equal
the oracle's (score desc, index asc) selection bit for bit, including ties, masks,
padding and negative, infinite and signed-zero scores."""
import numpy as np
import pytest
import torch

import lightning_indexer_top_amd as li
import oracle
from helpers import dev

pytestmark = pytest.mark.gpu


def check(scores, k, nv=None):
    g_idx, g_val = li.topk_select(dev(scores), k, dev(nv) if nv is not None else None)
    torch.cuda.synchronize()
    o_idx, o_val = oracle.topk(scores.astype(np.float64), k, nv)
    g_idx = g_idx.cpu().numpy()
    g_val = g_val.cpu().numpy().astype(np.float64)
    assert np.array_equal(g_idx, o_idx)
    fin = o_idx >= 0
    assert np.array_equal(g_val[fin], o_val[fin])
    assert np.isneginf(g_val[~fin]).all()


@pytest.mark.parametrize("S,k", [(1, 1), (7, 3), (100, 100), (1000, 64), (4097, 512), (5000, 2048), (3000, 2048)])
def test_random_rows(S, k):
    print("topk", S, k, flush=True)
    rng = np.random.default_rng(S + k)
    check(rng.standard_normal((5, S)).astype(np.float32), k)


def test_heavy_ties_and_masks():
    print("topk ties", flush=True)
    rng = np.random.default_rng(1)
    R, S = 9, 6000
    s = rng.integers(-20, 20, (R, S)).astype(np.float32)
    s[0] = 1.0                      # all equal
    s[1, ::3] = -np.inf             # infinities
    s[2] = -np.abs(s[2]) - 1        # all negative
    s[3, :100] = 0.0                # signed zeros among ties
    s[3, 100:200] = -0.0
    nv = np.array([6000, 6000, 6000, 6000, 0, 1, 511, 513, 7000], np.int32)
    for k in (1, 32, 512, 2048):
        check(s, k, nv)


def test_large_row_decode_shape():
    print("topk 131072", flush=True)
    rng = np.random.default_rng(2)
    check(rng.standard_normal((3, 131072)).astype(np.float32), 512)


def test_few_long_rows_multi_workgroup_path():
    # few rows of >= 16384 entries take the many-workgroups-per-row path: random
    # rows, heavy ties, a cut bin larger than the candidate list (whole-row
    # fallback), visible counts below k and zero
    print("topk multi-workgroup", flush=True)
    rng = np.random.default_rng(4)
    R, S = 7, 40000
    s = rng.standard_normal((R, S)).astype(np.float32)
    s[1] = 3.0                                         # all equal: cut bin overflows
    s[2] = rng.integers(0, 6, S).astype(np.float32)    # 6 distinct values
    s[3] = np.abs(s[3]) * 1e-30                        # tiny values
    s[4, 1000:] = -np.inf
    nv = np.array([40000, 39000, 40000, 20001, 40000, 300, 0], np.int32)
    for k in (1, 64, 512, 2048):
        check(s, k, nv)
        check(s, k)


def test_multi_workgroup_wide_select_edges():
    # the final pass of the multi-workgroup path resolves only the bits in which its
    # candidates differ: candidates over 60 binades of both signs, neighbours one
    # ulp apart, a single distinct value above a sea of ties, signed zeros at the
    # cut, and rows whose candidates straddle zero
    print("topk wide select", flush=True)
    rng = np.random.default_rng(9)
    R, S = 6, 50000
    s = np.empty((R, S), np.float32)
    s[0] = (rng.standard_normal(S) * 10.0 ** rng.uniform(-30, 30, S)).astype(np.float32)
    s[1] = np.float32(1.5) + np.arange(S, dtype=np.float32) * np.float32(2 ** -23)
    s[2] = 7.0
    s[2, rng.integers(0, S, 100)] = 7.5
    s[3] = -np.abs(rng.standard_normal(S)).astype(np.float32)
    s[3, :3000] = 0.0
    s[3, 3000:6000] = -0.0
    s[4] = rng.standard_normal(S).astype(np.float32) * 1e-3
    s[5] = rng.integers(-3, 3, S).astype(np.float32) * np.float32(2 ** -20)
    for k in (1, 100, 512, 2048):
        check(s, k)
