"""Pins of the oracle's paged-cache reads ("Long context" lecture, section
"Sparsity Is a Systems Feature: The Blast Radius", paragraph "KV-cache
management": indexer keys and scales in pages of 64, the latent read at page size
1).  A pool is built by scattering contiguous per-sequence rows into randomly
chosen pages; reading it back through the table must give the rows, and the
paged score and attention must equal the unpaged oracle on them."""
import numpy as np

import oracle
import synth

PAGE = 64


def scatter_pages(rows, extra_pages, seed):
    """rows [B, S, ...] -> (pool [num_pages, 64, ...], table [B, max_pages]) with the
    pages in a random order among extra garbage pages."""
    B, S = rows.shape[:2]
    P = (S + PAGE - 1) // PAGE
    rng = np.random.default_rng(seed)
    num = B * P + extra_pages
    perm = rng.permutation(num)[:B * P].reshape(B, P)
    pool = rng.integers(0, 255, (num, PAGE) + rows.shape[2:]).astype(rows.dtype)
    for b in range(B):
        for p in range(P):
            n = min(PAGE, S - p * PAGE)
            pool[perm[b, p], :n] = rows[b, p * PAGE:p * PAGE + n]
    table = np.concatenate([perm, rng.integers(0, num, (B, 3))], axis=1).astype(np.int32)  # unused tail entries
    return pool, table


def test_unpage_inverts_the_scatter():
    rows = synth.normal_bf16(0x5EED0C00, 3, (3, 1000, 8))
    pool, table = scatter_pages(rows, 7, 0)
    assert np.array_equal(oracle.unpage(pool, table, 1000), rows)
    scales = synth.uniform_f32(0x5EED0C00, 4, (3, 1000), 0.5, 2.0)
    spool, stab = scatter_pages(scales, 2, 1)
    assert np.array_equal(oracle.unpage(spool, stab, 1000), scales)


def test_paged_score_equals_unpaged():
    B, T, S, H = 2, 2, 700, 8
    codes, sc = synth.fp8_rows(0x5EED0C01, 3, B * S, 128)
    codes, sc = codes.reshape(B, S, 128), sc.reshape(B, S)
    q = synth.normal_bf16(0x5EED0C01, 1, (B, T, H, 128), 0.1)
    w = synth.uniform_f32(0x5EED0C01, 2, (B, T, H))
    rng = np.random.default_rng(2)
    P = (S + PAGE - 1) // PAGE
    perm = rng.permutation(B * P + 5)[:B * P].reshape(B, P).astype(np.int32)
    kpool = rng.integers(0, 120, (B * P + 5, PAGE, 128)).astype(np.uint8)
    spool = rng.uniform(0.1, 1, (B * P + 5, PAGE)).astype(np.float32)
    for b in range(B):
        for p in range(P):
            n = min(PAGE, S - p * PAGE)
            kpool[perm[b, p], :n] = codes[b, p * PAGE:p * PAGE + n]
            spool[perm[b, p], :n] = sc[b, p * PAGE:p * PAGE + n]
    nv = np.array([700, 65, 0, 300], np.int32)
    got = oracle.indexer_score_paged(q, oracle.BF16, w, kpool, spool, perm, S, nv)
    ref = oracle.indexer_score(q, oracle.BF16, w, codes, oracle.FP8_E4M3, sc, nv)
    assert np.array_equal(got, ref)


def test_paged_attention_equals_unpaged():
    B, Hq, S, k, dqk, dv = 2, 4, 300, 20, 24, 16
    kv = synth.normal_bf16(0x5EED0C02, 5, (B, S, dqk))
    q = synth.normal_bf16(0x5EED0C02, 6, (B, Hq, dqk))
    rng = np.random.default_rng(3)
    slots = rng.permutation(B * S + 50)[:B * S].reshape(B, S)
    pool = rng.integers(0, 65535, (B * S + 50, dqk)).astype(np.uint16)
    for b in range(B):
        pool[slots[b]] = kv[b]
    idx = np.stack([rng.choice(S, k, replace=False) for _ in range(B)]).astype(np.int32)
    idx[0, 3] = -1
    idx[1, 7] = S + 4  # out of range: selects nothing
    o1, l1 = oracle.sparse_attn_paged(q, pool, slots.astype(np.int32), idx, dv, 0.2)
    idx2 = np.where((idx >= 0) & (idx < S), idx, -1)
    o2, l2 = oracle.sparse_attn(q, kv, idx2, dv, 0.2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
