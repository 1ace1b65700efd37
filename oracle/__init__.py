"""fp64 CPU oracle of the lightning-indexer hot path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this
package.  It wraps liboracle.so (oracle.c), which shares no code with the GPU
library.  Array arguments are numpy arrays holding the same bytes the GPU path
receives (fp32, bf16 bit patterns as uint16, fp8 E4M3FN codes as uint8, int8).
"""
import ctypes
import os

import numpy as np

F32, BF16, FP8_E4M3, I8 = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None
_i64 = ctypes.c_int64
_ptr = ctypes.c_void_p


def lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(path)
        L.orc_dec_bf16.argtypes = [ctypes.c_uint16]
        L.orc_dec_bf16.restype = ctypes.c_double
        L.orc_dec_e4m3.argtypes = [ctypes.c_uint8]
        L.orc_dec_e4m3.restype = ctypes.c_double
        L.orc_threads_used.restype = ctypes.c_int
        L.orc_indexer_score.argtypes = [_ptr, ctypes.c_int, _ptr, _ptr, ctypes.c_int, _ptr, _ptr,
                                        _i64, _i64, _i64, _i64, _i64, _ptr]
        L.orc_indexer_score.restype = None
        L.orc_topk.argtypes = [_ptr, _ptr, _i64, _i64, _i64, _ptr, _ptr]
        L.orc_topk.restype = None
        L.orc_compact_query.argtypes = [_ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, _ptr, _ptr, _ptr]
        L.orc_compact_query.restype = None
        L.orc_compact_search.argtypes = [_ptr] * 7 + [_i64] * 7 + [_ptr] * 4
        L.orc_compact_search.restype = None
        L.orc_sparse_attn_rows.argtypes = [_ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, _i64, ctypes.c_double,
                                           _ptr, _ptr]
        L.orc_sparse_attn_rows.restype = None
        L.orc_sparse_attn.argtypes = [_ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, _i64, _i64, ctypes.c_double,
                                      _ptr, _ptr]
        L.orc_sparse_attn.restype = None
        L.orc_pq_query.argtypes = [_ptr, _ptr, ctypes.c_double, _i64, _i64, _i64, _ptr, _ptr]
        L.orc_pq_query.restype = None
        L.orc_pq_search.argtypes = [_ptr, _ptr, _ptr, ctypes.c_double, _ptr, _ptr, _ptr] + [_i64] * 6 + [_ptr] * 4
        L.orc_pq_search.restype = None
        L.orc_e4m3_rne.argtypes = [ctypes.c_float]
        L.orc_e4m3_rne.restype = ctypes.c_uint8
        L.orc_pool_keys.argtypes = [_ptr, _i64, _i64, _i64, _i64, _ptr, _ptr]
        L.orc_pool_keys.restype = None
        L.orc_pooled_select.argtypes = [_ptr, ctypes.c_int, _ptr, _ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, _i64,
                                        _i64, _i64, _ptr, _ptr]
        L.orc_pooled_select.restype = None
        _LIB = L
    return _LIB


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


_DT = {F32: np.float32, BF16: np.uint16, FP8_E4M3: np.uint8, I8: np.int8}


def threads_used() -> int:
    """Threads the last multi-row oracle call ran on."""
    return int(lib().orc_threads_used())


def dec_bf16(b: int) -> float:
    return float(lib().orc_dec_bf16(int(b)))


def dec_e4m3(c: int) -> float:
    return float(lib().orc_dec_e4m3(int(c)))


def indexer_score(q, q_type, w, k, k_type, k_scale=None, nv=None):
    """Scores [B*T, S] (fp64) of q [B, T, H, d], w [B, T, H], k [B, S, d].
    Keys s >= nv[row] score -inf."""
    q = _c(q, _DT[q_type]); k = _c(k, _DT[k_type]); w = _c(w, np.float32)
    k_scale = _c(k_scale, np.float32); nv = _c(nv, np.int32)
    B, T, H, d = q.shape
    S = k.shape[1]
    assert k.shape == (B, S, d) and w.shape == (B, T, H)
    assert k_scale is None or k_scale.shape == (B, S)
    assert nv is None or nv.size == B * T
    out = np.empty((B * T, S), np.float64)
    lib().orc_indexer_score(_p(q), q_type, _p(w), _p(k), k_type, _p(k_scale), _p(nv), B, T, S, H, d, _p(out))
    return out


def topk(scores, k, nv=None):
    """(idx int32 [R, k], val fp64 [R, k]): the k best by (score desc, index asc),
    listed in ascending index order, padded with (-1, -inf)."""
    scores = _c(scores, np.float64)
    R, S = scores.shape
    nv = _c(nv, np.int32)
    idx = np.empty((R, k), np.int32)
    val = np.empty((R, k), np.float64)
    lib().orc_topk(_p(scores), _p(nv), R, S, k, _p(idx), _p(val))
    return idx, val


def compact_query(q, w, P):
    """(q8 [B, H, dc] int8, qs [B, H] fp64, W [B, H] fp64) of bf16 queries q [B, H, d]."""
    q = _c(q, np.uint16); w = _c(w, np.float32); P = _c(P, np.float32)
    B, H, d = q.shape
    dc = P.shape[0]
    q8 = np.empty((B, H, dc), np.int8)
    qs = np.empty((B, H), np.float64)
    W = np.empty((B, H), np.float64)
    lib().orc_compact_query(_p(q), _p(w), _p(P), B, H, d, dc, _p(q8), _p(qs), _p(W))
    return q8, qs, W


def compact_search(q, w, P, c, cs, k_full, m, k, nv=None, want_s1=False):
    """Two-stage search -> dict(shortlist [B, m], idx [B, k], val [B, k], s1 [B, S] or None)."""
    q = _c(q, np.uint16); w = _c(w, np.float32); P = _c(P, np.float32)
    c = _c(c, np.int8); cs = _c(cs, np.float32); k_full = _c(k_full, np.uint16); nv = _c(nv, np.int32)
    B, H, d = q.shape
    S = c.shape[1]
    dc = P.shape[0]
    assert c.shape == (B, S, dc) and cs.shape == (B, S) and k_full.shape == (B, S, d)
    assert dc <= 256
    sl = np.empty((B, m), np.int32)
    idx = np.empty((B, k), np.int32)
    val = np.empty((B, k), np.float64)
    s1 = np.empty((B, S), np.float64) if want_s1 else None
    lib().orc_compact_search(_p(q), _p(w), _p(P), _p(c), _p(cs), _p(k_full), _p(nv), B, S, H, d, dc, m, k,
                             _p(sl), _p(idx), _p(val), _p(s1))
    return {"shortlist": sl, "idx": idx, "val": val, "s1": s1}


def sparse_attn_rows(q, rows, idx, dv, tau):
    """q [B, Hq, dqk] bf16, rows [B, k, dqk] bf16 (gathered), idx [B, k] -> (out [B, Hq, dv], lse [B, Hq])."""
    q = _c(q, np.uint16); rows = _c(rows, np.uint16); idx = _c(idx, np.int32)
    B, Hq, dqk = q.shape
    k = idx.shape[1]
    assert rows.shape == (B, k, dqk)
    out = np.empty((B, Hq, dv), np.float64)
    lse = np.empty((B, Hq), np.float64)
    lib().orc_sparse_attn_rows(_p(q), _p(rows), _p(idx), B, Hq, k, dqk, dv, tau, _p(out), _p(lse))
    return out, lse


def sparse_attn(q, kv, idx, dv, tau):
    """q [B, Hq, dqk], kv [B, S, dqk] bf16, idx [B, k] in [-1, S) -> (out, lse)."""
    q = _c(q, np.uint16); kv = _c(kv, np.uint16); idx = _c(idx, np.int32)
    B, Hq, dqk = q.shape
    S = kv.shape[1]
    k = idx.shape[1]
    assert idx.min() >= -1 and idx.max() < S
    out = np.empty((B, Hq, dv), np.float64)
    lse = np.empty((B, Hq), np.float64)
    lib().orc_sparse_attn(_p(q), _p(kv), _p(idx), B, Hq, S, k, dqk, dv, tau, _p(out), _p(lse))
    return out, lse


def e4m3_rne(x: float) -> int:
    """OCP E4M3FN code nearest the fp32 value x (ties to even, saturating)."""
    return int(lib().orc_e4m3_rne(float(x)))


def pool_keys(k, pool):
    """Pooled fp8 keys of bf16 token keys k [B, L, d] (uint16): (codes uint8
    [B, L // pool, d], scales float32 [B, L // pool])."""
    k = _c(k, np.uint16)
    B, L, d = k.shape
    Sp = L // pool
    codes = np.empty((B, Sp, d), np.uint8)
    scales = np.empty((B, Sp), np.float32)
    lib().orc_pool_keys(_p(k), B, L, d, pool, _p(codes), _p(scales))
    return codes, scales


def pooled_select(q, q_type, w, codes, scales, pool, k, nv_tokens=None):
    """(idx_tokens int32 [B*T, k * pool], val_blocks fp64 [B*T, k]): the top-k pooled
    blocks of q [B, T, H, d], w [B, T, H] over codes [B, Sp, d] + scales [B, Sp],
    each expanded to its pool tokens."""
    q = _c(q, _DT[q_type]); w = _c(w, np.float32); codes = _c(codes, np.uint8); scales = _c(scales, np.float32)
    nv_tokens = _c(nv_tokens, np.int32)
    B, T, H, d = q.shape
    Sp = codes.shape[1]
    assert codes.shape == (B, Sp, d) and scales.shape == (B, Sp) and w.shape == (B, T, H)
    assert nv_tokens is None or nv_tokens.size == B * T
    idx = np.empty((B * T, k * pool), np.int32)
    val = np.empty((B * T, k), np.float64)
    lib().orc_pooled_select(_p(q), q_type, _p(w), _p(codes), _p(scales), _p(nv_tokens), B, T, Sp, H, d, pool, k,
                            _p(idx), _p(val))
    return idx, val


# ---- paged caches ("Long context", section "Sparsity Is a Systems Feature: The
# Blast Radius", paragraph "KV-cache management": indexer keys and their scales in
# separate buffers read in pages of 64, the latent read at page size 1) --------

def unpage(pool, table, S):
    """Logical rows [B, S, ...] of a paged pool [num_pages, page, ...]: row s of
    sequence b is pool[table[b, s // page], s % page]."""
    pool = np.asarray(pool)
    table = np.asarray(table, np.int64)
    page = pool.shape[1]
    s = np.arange(S, dtype=np.int64)
    return pool[table[:, s // page], s % page]


def indexer_score_paged(q, q_type, w, k_pool, k_scale_pool, page_table, S, nv=None):
    """O1 over paged fp8 keys: the keys gathered through the page table, then scored."""
    return indexer_score(q, q_type, w, unpage(k_pool, page_table, S), FP8_E4M3,
                         unpage(k_scale_pool, page_table, S), nv)


def sparse_attn_paged(q, kv_pool, slot_table, idx, dv, tau):
    """O4 over a latent pool read at page size 1: row idx[b, i] of sequence b is
    kv_pool[slot_table[b, idx[b, i]]]; entries outside [0, S) select nothing."""
    idx = np.asarray(idx, np.int64)
    slot_table = np.asarray(slot_table, np.int64)
    S = slot_table.shape[1]
    ok = (idx >= 0) & (idx < S)
    slots = np.where(ok, np.take_along_axis(slot_table, np.where(ok, idx, 0), axis=1), 0)
    rows = np.asarray(kv_pool)[slots]
    rows[~ok] = 0
    return sparse_attn_rows(q, rows, np.where(ok, idx, -1).astype(np.int32), dv, tau)


def pq_query(q, w, sigma):
    """(q8 [B, H, d] int8, W [B, H] fp64): the int8 query codes of the product-
    quantised search and the head weights W = (w * qs) * sigma."""
    q = _c(q, np.uint16); w = _c(w, np.float32)
    B, H, d = q.shape
    q8 = np.empty((B, H, d), np.int8)
    W = np.empty((B, H), np.float64)
    lib().orc_pq_query(_p(q), _p(w), float(sigma), B, H, d, _p(q8), _p(W))
    return q8, W


def pq_search(q, w, cb, sigma, codes, k_full, m, k, nv=None, want_s1=False):
    """Two-stage search over product-quantised keys -> dict(shortlist [B, m],
    idx [B, k], val [B, k], s1 [B, S] or None).  cb [d/4, 256, 4] int8 codebook,
    sigma its scale, codes [B, S, d/4] uint8, k_full [B, S, d] bf16."""
    q = _c(q, np.uint16); w = _c(w, np.float32); cb = _c(cb, np.int8); codes = _c(codes, np.uint8)
    k_full = _c(k_full, np.uint16); nv = _c(nv, np.int32)
    B, H, d = q.shape
    S = codes.shape[1]
    assert cb.shape == (d // 4, 256, 4) and codes.shape == (B, S, d // 4) and k_full.shape == (B, S, d)
    sl = np.empty((B, m), np.int32)
    idx = np.empty((B, k), np.int32)
    val = np.empty((B, k), np.float64)
    s1 = np.empty((B, S), np.float64) if want_s1 else None
    lib().orc_pq_search(_p(q), _p(w), _p(cb), float(sigma), _p(codes), _p(k_full), _p(nv), B, S, H, d, m, k,
                        _p(sl), _p(idx), _p(val), _p(s1))
    return {"shortlist": sl, "idx": idx, "val": val, "s1": s1}

