"""Pins of the oracle's pooled-key indexer (O6): keys pooled four at a time
("Long context" lecture, section "The 2025-2026 Hybrid Turn: Linear Attention
Returns": IndexPool, four indexer keys pooled into one, index_kpool = 4) and
scored by 32 heads of 128 dims with the top blocks expanded back to tokens
("Latent Sparse Attention", section "Where the time goes").  The pins are
independent of the oracle's code: torch's own fp8 conversion, numpy float32
arithmetic for the pooling, numpy fp64 brute force for the selection."""
import numpy as np
import pytest
import torch

import oracle
import synth

E4M3 = torch.float8_e4m3fn


def torch_e4m3(x):
    """Codes of fp32 values under torch's float8_e4m3fn conversion (round to nearest
    even)."""
    return torch.from_numpy(np.asarray(x, np.float32)).to(E4M3).view(torch.uint8).numpy()


def test_e4m3_encoder_matches_torch():
    # every finite code, the midpoints between neighbours (ties), values just off
    # them, subnormals and zero, both signs
    vals = torch.arange(0, 0x7F, dtype=torch.uint8).view(E4M3).to(torch.float64).numpy()
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(0)
    x = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9), rng.uniform(0, 448, 3000),
                        rng.uniform(0, 0.02, 1000), [0.0]]).astype(np.float32)
    x = np.concatenate([x, -x])
    got = np.array([oracle.e4m3_rne(v) for v in x], np.uint8)
    assert np.array_equal(got, torch_e4m3(x))
    # saturation: values past the largest finite code keep its magnitude
    assert oracle.e4m3_rne(470.0) == 0x7E and oracle.e4m3_rne(-1e30) == 0xFE


def numpy_pool(k_bf16, pool):
    """The pooling definition in numpy float32: sequential sum, times 1/pool, amax /
    448 scale, fp32 division, codes from torch's conversion."""
    kf = (k_bf16.astype(np.uint32) << 16).view(np.float32)
    B, L, d = kf.shape
    Sp = L // pool
    blocks = kf[:, :Sp * pool].reshape(B, Sp, pool, d)
    s = blocks[:, :, 0].copy()
    for t in range(1, pool):
        s = (s + blocks[:, :, t]).astype(np.float32)
    m = (s * np.float32(1.0 / pool)).astype(np.float32)
    amax = np.abs(m).max(axis=-1)
    sc = np.where(amax > 0, (amax / np.float32(448.0)).astype(np.float32), np.float32(1.0)).astype(np.float32)
    return torch_e4m3((m / sc[..., None]).astype(np.float32)), sc


@pytest.mark.parametrize("pool", [1, 2, 4, 8])
def test_pooling_matches_numpy_float32(pool):
    k = synth.normal_bf16(0x5EED0900 + pool, 3, (2, 8 * 9 + 3, 128))  # an incomplete last block
    codes, scales = oracle.pool_keys(k, pool)
    rc, rs = numpy_pool(k, pool)
    assert codes.shape == (2, (8 * 9 + 3) // pool, 128)
    assert np.array_equal(scales, rs)
    assert np.array_equal(codes, rc)


def test_identical_keys_pool_to_the_key():
    # four copies of one key pool to that key's own fp8 encoding; a zero block gives
    # zero codes with scale 1
    k1 = synth.normal_bf16(0x5EED0901, 3, (1, 1, 128))
    k = np.repeat(k1, 4, axis=1)
    k = np.concatenate([k, np.zeros((1, 4, 128), np.uint16)], axis=1)
    codes, scales = oracle.pool_keys(k, 4)
    c1, s1 = oracle.pool_keys(k1, 1)
    assert np.array_equal(codes[0, 0], c1[0, 0]) and scales[0, 0] == s1[0, 0]
    assert (codes[0, 1] == 0).all() and scales[0, 1] == 1.0
    # the decoded pooled key is within half an fp8 step of the fp64 mean
    kk = synth.normal_bf16(0x5EED0902, 3, (1, 4, 128))
    c, s = oracle.pool_keys(kk, 4)
    mean = ((kk.astype(np.uint32) << 16).view(np.float32).astype(np.float64)).mean(axis=1)[0]
    dec = torch.from_numpy(c[0]).view(E4M3).to(torch.float64).numpy() * float(s[0, 0])
    assert np.all(np.abs(dec - mean) <= np.abs(mean) * 2.0 ** -4 + float(s[0, 0]) * 2.0 ** -10 + 1e-7)


def brute_pooled(q, w, codes, scales, pool, k, nv_tokens):
    """numpy fp64: decode the pooled keys, score every visible complete block, sort by
    (score desc, block asc), keep k, list them ascending, expand to tokens."""
    B, T, H, d = q.shape
    Sp = codes.shape[1]
    qf = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    kd = torch.from_numpy(codes).view(E4M3).to(torch.float64).numpy() * scales.astype(np.float64)[..., None]
    idx = np.full((B * T, k * pool), -1, np.int32)
    val = np.full((B * T, k), -np.inf)
    for b in range(B):
        for t in range(T):
            r = b * T + t
            n = Sp if nv_tokens is None else min(max(int(nv_tokens[r]), 0) // pool, Sp)
            dots = qf[b, t] @ kd[b, :n].T                       # [H, n]
            sc = (w[b, t].astype(np.float64)[:, None] * np.maximum(dots, 0)).sum(0)
            order = np.lexsort((np.arange(n), -sc))[:k]
            sel = np.sort(order)
            val[r, :len(sel)] = sc[sel]
            for j, bj in enumerate(sel):
                idx[r, j * pool:(j + 1) * pool] = bj * pool + np.arange(pool)
    return idx, val


@pytest.mark.parametrize("pool,k", [(4, 16), (4, 40), (2, 7), (1, 12)])
def test_pooled_selection_brute_force(pool, k):
    B, T, L, H = 2, 3, 4 * 37 + 2, 32
    k_tok = synth.normal_bf16(0x5EED0910 + pool, 3, (B, L, 128))
    q = synth.normal_bf16(0x5EED0910 + pool, 1, (B, T, H, 128), 1 / np.sqrt(128))
    w = synth.uniform_f32(0x5EED0910 + pool, 2, (B, T, H))
    codes, scales = oracle.pool_keys(k_tok, pool)
    nv = np.array([L, 0, pool * 5 + pool - 1, 3, L - 1, pool * 20], np.int32)
    for nvt in (None, nv):
        idx, val = oracle.pooled_select(q, oracle.BF16, w, codes, scales, pool, k, nvt)
        ri, rv = brute_pooled(q, w, codes, scales, pool, k, nvt)
        assert np.array_equal(idx, ri)
        fin = np.isfinite(rv)
        assert np.array_equal(np.isfinite(val), fin)
        np.testing.assert_allclose(val[fin], rv[fin], rtol=1e-12)
    # a row that sees no complete block selects nothing; a block completed by its
    # last token is visible, one short of it is not
    idx, _ = oracle.pooled_select(q, oracle.BF16, w, codes, scales, pool, k, nv)
    assert (idx[1] == -1).all()
    assert idx[2].max() == 5 * pool - 1                      # nv = 6 pool - 1: blocks 0..4 visible
    if 3 // pool == 0:
        assert (idx[3] == -1).all()                           # nv = 3 < pool: no complete block
    else:
        assert idx[3].max() == (3 // pool) * pool - 1
