"""Python binding of the gfx950 lightning-indexer library (liblightning_indexer.so).

Argument marshalling only: every step runs in the library's HIP kernels, enqueued
on torch's current stream.  torch provides device memory and streams.  The
functions mirror the C entry points of include/li.h:

    indexer_score          scores of every key for every query row
    topk_select            the k best keys per row, listed in ascending key index
    indexer_topk           scoring + selection without returning the scores
    compact_search_rerank  compact-key shortlist + exact rerank
    sparse_attn_gather     attention over only the selected latent rows

If the library is missing these raise; there is no fallback.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblightning_indexer.so")

LI_F32, LI_BF16, LI_FP8_E4M3, LI_I8 = 0, 1, 2, 3
TOPK_MAX = 2048

_STATUS = {0: "LI_OK", 1: "LI_ERR_NULL", 2: "LI_ERR_SHAPE", 3: "LI_ERR_DTYPE", 4: "LI_ERR_ALIGN",
           5: "LI_ERR_WORKSPACE", 6: "LI_ERR_LAUNCH"}

_LIB = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_Z = ctypes.c_size_t


class LIError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = lib().li_last_error().decode(errors="replace")
        super().__init__(f"{where}: {_STATUS.get(status, status)}: {msg}")


def lib():
    """Load the HIP library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.li_status_string.argtypes = [_I]
        L.li_status_string.restype = ctypes.c_char_p
        L.li_last_error.restype = ctypes.c_char_p
        L.li_version.restype = ctypes.c_char_p
        L.li_indexer_score.argtypes = [_P, _I, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _P, _P]
        L.li_topk_workspace_bytes.argtypes = [_I, _I, _I]
        L.li_topk_workspace_bytes.restype = _Z
        L.li_topk_select.argtypes = [_P, _P, _I, _I, _I, _P, _P, _P, _Z, _P]
        L.li_topk_select_noalloc.argtypes = [_P, _P, _I, _I, _I, _P, _P, _P]
        L.li_indexer_topk_workspace_bytes.argtypes = [_I, _I, _I, _I, _I, _I, _I]
        L.li_indexer_topk_workspace_bytes.restype = _Z
        L.li_indexer_topk.argtypes = [_P, _I, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _Z, _P]
        L.li_compact_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
        L.li_compact_workspace_bytes.restype = _Z
        L.li_compact_search_rerank.argtypes = [_P] * 7 + [_I] * 7 + [_P] * 4 + [_Z, _P]
        L.li_sparse_attn_workspace_bytes.argtypes = [_I, _I, _I, _I]
        L.li_sparse_attn_workspace_bytes.restype = _Z
        L.li_sparse_attn_gather.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P, _P, _P, _Z, _P]
        L.li_pool_keys.argtypes = [_P, _I, _I, _I, _I, _I, _P, _P, _P]
        L.li_pooled_indexer_topk_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
        L.li_pooled_indexer_topk_workspace_bytes.restype = _Z
        L.li_pooled_indexer_topk.argtypes = [_P, _I, _P, _P, _P, _P] + [_I] * 7 + [_P, _P, _P, _Z, _P]
        L.li_layer_stream_buffer_bytes.argtypes = [_I, _Z]
        L.li_layer_stream_buffer_bytes.restype = _Z
        L.li_layer_stream_prefill.argtypes = [_P, _P, _P, _P, _P, _Z, _P, _P, _I, _P, _P, _Z] + [_I] * 6 + [_P, _P, _P,
                                                                                                         _P]
        L.li_pq_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
        L.li_pq_workspace_bytes.restype = _Z
        L.li_pq_search_rerank.argtypes = [_P, _P, _P, ctypes.c_float, _P, _P, _P] + [_I] * 6 + [_P] * 4 + [_Z, _P]
        L.li_indexer_score_paged.argtypes = [_P, _I, _P, _P, _P, _P, _I, _I, _I, _P] + [_I] * 5 + [_P, _P]
        L.li_indexer_topk_paged_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
        L.li_indexer_topk_paged_workspace_bytes.restype = _Z
        L.li_indexer_topk_paged.argtypes = [_P, _I, _P, _P, _P, _P, _I, _I, _I, _P] + [_I] * 6 + [_P, _P, _P, _Z, _P]
        L.li_sparse_attn_gather_paged.argtypes = [_P, _P, _P, _I, _I, _P, _I, _I, _I, _I, _I, _I, ctypes.c_float, _P,
                                                  _P, _P]
        for name in ("li_indexer_score", "li_topk_select", "li_topk_select_noalloc", "li_indexer_topk",
                     "li_pool_keys", "li_pooled_indexer_topk", "li_indexer_score_paged", "li_indexer_topk_paged",
                     "li_sparse_attn_gather_paged", "li_pq_search_rerank", "li_layer_stream_prefill", "li_compact_search_rerank",
                     "li_sparse_attn_gather"):
            getattr(L, name).restype = _I
        _LIB = L
    return _LIB


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t, name):
    if not (isinstance(t, torch.Tensor) and t.is_cuda):
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _dtype_code(t, name):
    if t.dtype == torch.float32:
        return LI_F32
    if t.dtype == torch.bfloat16:
        return LI_BF16
    if t.dtype == torch.float8_e4m3fn:
        return LI_FP8_E4M3
    if t.dtype == torch.int8:
        return LI_I8
    raise TypeError(f"{name}: unsupported dtype {t.dtype}")


def _check(status, where):
    if status != 0:
        raise LIError(status, where)


def _workspace(nbytes, device, workspace=None, zeroed=True):
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace needs {nbytes} bytes")
        return workspace, workspace.numel() * workspace.element_size()
    # zero-filled unless the caller says otherwise: the fused decode selection keeps
    # per-row counters there, which a zeroed workspace has ready (any contents give
    # the same results)
    if zeroed:
        return torch.zeros(nbytes, dtype=torch.uint8, device=device), nbytes
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def indexer_score(q, w, k, k_scale=None, nv=None, out=None):
    """Scores [B*T, S] fp32 of q [B, T, H, 128] (bf16/fp32), w [B, T, H] fp32 against
    k [B, S, 128] (float8_e4m3fn with k_scale [B, S], bf16 or fp32).  nv [B*T] int32
    limits each row to keys s < nv[row]; invisible keys score -inf."""
    _dev(q, "q"); _dev(w, "w"); _dev(k, "k")
    B, T, H, d = q.shape
    S = k.shape[1]
    if k_scale is not None:
        _dev(k_scale, "k_scale")
    if nv is not None:
        _dev(nv, "nv")
    if out is None:
        out = torch.empty((B * T, S), dtype=torch.float32, device=q.device)
    st = lib().li_indexer_score(_ptr(q), _dtype_code(q, "q"), _ptr(w), _ptr(k), _dtype_code(k, "k"), _ptr(k_scale),
                                _ptr(nv), B, T, S, H, d, _ptr(out), _stream(q.device))
    _check(st, "li_indexer_score")
    return out


def topk_workspace_bytes(R, S, k):
    return int(lib().li_topk_workspace_bytes(R, S, k))


def topk_select(scores, k, nv=None, with_values=True, workspace=None, out=None):
    """(idx [R, k] int32, val [R, k] fp32 or None) of scores [R, S]."""
    _dev(scores, "scores")
    R, S = scores.shape
    if out is None:
        idx = torch.empty((R, k), dtype=torch.int32, device=scores.device)
        val = torch.empty((R, k), dtype=torch.float32, device=scores.device) if with_values else None
    else:
        idx, val = out
    # every byte of this workspace is written before it is read
    ws, nb = _workspace(lib().li_topk_workspace_bytes(R, S, k), scores.device, workspace, zeroed=False)
    st = lib().li_topk_select(_ptr(scores), _ptr(nv), R, S, k, _ptr(idx), _ptr(val), _ptr(ws), nb,
                              _stream(scores.device))
    _check(st, "li_topk_select")
    return idx, val


def topk_select_noalloc(scores, k, nv=None, with_values=True, out=None):
    """topk_select without a workspace: the library's static per-GPU scratch serves
    the few-long-rows path (li_topk_select_noalloc; calls on one GPU must not
    overlap)."""
    _dev(scores, "scores")
    R, S = scores.shape
    if out is None:
        idx = torch.empty((R, k), dtype=torch.int32, device=scores.device)
        val = torch.empty((R, k), dtype=torch.float32, device=scores.device) if with_values else None
    else:
        idx, val = out
    st = lib().li_topk_select_noalloc(_ptr(scores), _ptr(nv), R, S, k, _ptr(idx), _ptr(val), _stream(scores.device))
    _check(st, "li_topk_select_noalloc")
    return idx, val


def indexer_topk_workspace_bytes(q_type, k_type, B, T, S, H, topk):
    """Workspace bytes li_indexer_topk needs for these dtype codes and shape."""
    return int(lib().li_indexer_topk_workspace_bytes(q_type, k_type, B, T, S, H, topk))


def indexer_topk(q, w, k, topk, k_scale=None, nv=None, with_values=True, workspace=None, out=None):
    """(idx [B*T, topk] int32, val [B*T, topk] fp32 or None): scoring + selection."""
    _dev(q, "q"); _dev(w, "w"); _dev(k, "k")
    B, T, H, d = q.shape
    S = k.shape[1]
    R = B * T
    if out is None:
        idx = torch.empty((R, topk), dtype=torch.int32, device=q.device)
        val = torch.empty((R, topk), dtype=torch.float32, device=q.device) if with_values else None
    else:
        idx, val = out
    ws, nb = _workspace(indexer_topk_workspace_bytes(_dtype_code(q, "q"), _dtype_code(k, "k"), B, T, S, H, topk),
                        q.device, workspace)
    st = lib().li_indexer_topk(_ptr(q), _dtype_code(q, "q"), _ptr(w), _ptr(k), _dtype_code(k, "k"), _ptr(k_scale),
                               _ptr(nv), B, T, S, H, d, topk, _ptr(idx), _ptr(val), _ptr(ws), nb, _stream(q.device))
    _check(st, "li_indexer_topk")
    return idx, val


def pool_keys(k, pool, out=None):
    """Pooled fp8 keys of bf16 token keys k [B, L, 128]: (codes float8_e4m3fn
    [B, L // pool, 128], scales fp32 [B, L // pool])."""
    _dev(k, "k")
    B, L, d = k.shape
    Sp = L // pool
    if out is None:
        codes = torch.empty((B, Sp, d), dtype=torch.float8_e4m3fn, device=k.device)
        scales = torch.empty((B, Sp), dtype=torch.float32, device=k.device)
    else:
        codes, scales = out
    st = lib().li_pool_keys(_ptr(k), _dtype_code(k, "k"), B, L, d, pool, _ptr(codes), _ptr(scales), _stream(k.device))
    _check(st, "li_pool_keys")
    return codes, scales


def pooled_indexer_topk_workspace_bytes(B, T, Sp, H, topk):
    return int(lib().li_pooled_indexer_topk_workspace_bytes(B, T, Sp, H, topk))


def pooled_indexer_topk(q, w, codes, scales, pool, topk, nv_tokens=None, with_values=True, workspace=None,
                        out=None):
    """(idx_tokens [B*T, topk*pool] int32, val_blocks [B*T, topk] fp32 or None): the top
    pooled blocks of q [B, T, H, 128] (bf16), w [B, T, H] over codes [B, Sp, 128]
    (float8_e4m3fn) + scales [B, Sp], expanded to token indices."""
    _dev(q, "q"); _dev(w, "w"); _dev(codes, "codes"); _dev(scales, "scales")
    B, T, H, d = q.shape
    Sp = codes.shape[1]
    R = B * T
    if out is None:
        idx = torch.empty((R, topk * pool), dtype=torch.int32, device=q.device)
        val = torch.empty((R, topk), dtype=torch.float32, device=q.device) if with_values else None
    else:
        idx, val = out
    ws, nb = _workspace(pooled_indexer_topk_workspace_bytes(B, T, Sp, H, topk), q.device, workspace)
    st = lib().li_pooled_indexer_topk(_ptr(q), _dtype_code(q, "q"), _ptr(w), _ptr(codes), _ptr(scales),
                                      _ptr(nv_tokens), B, T, Sp, H, d, pool, topk, _ptr(idx), _ptr(val), _ptr(ws), nb,
                                      _stream(q.device))
    _check(st, "li_pooled_indexer_topk")
    return idx, val


def compact_workspace_bytes(B, S, H, m, k):
    return int(lib().li_compact_workspace_bytes(B, S, H, m, k))


def compact_search_rerank(q, w, P, ck, ck_scale, k_full, m, k, nv=None, want_shortlist=True, workspace=None,
                          out=None):
    """Two-stage search.  q [B, H, 128] bf16, w [B, H], P [32, 128] fp32, ck [B, S, 32]
    int8, ck_scale [B, S], k_full [B, S, 128] bf16 -> (shortlist [B, m] or None,
    idx [B, k], val [B, k] fp64)."""
    for t, n in ((q, "q"), (w, "w"), (P, "P"), (ck, "ck"), (ck_scale, "ck_scale"), (k_full, "k_full")):
        _dev(t, n)
    B, H, d = q.shape
    S, dc = ck.shape[1], ck.shape[2]
    if out is None:
        sl = torch.empty((B, m), dtype=torch.int32, device=q.device) if want_shortlist else None
        idx = torch.empty((B, k), dtype=torch.int32, device=q.device)
        val = torch.empty((B, k), dtype=torch.float64, device=q.device)
    else:
        sl, idx, val = out
    ws, nb = _workspace(compact_workspace_bytes(B, S, H, m, k), q.device, workspace)
    st = lib().li_compact_search_rerank(_ptr(q), _ptr(w), _ptr(P), _ptr(ck), _ptr(ck_scale), _ptr(k_full), _ptr(nv),
                                        B, S, H, d, dc, m, k, _ptr(sl), _ptr(idx), _ptr(val), _ptr(ws), nb,
                                        _stream(q.device))
    _check(st, "li_compact_search_rerank")
    return sl, idx, val


def pq_workspace_bytes(B, S, H, m, k):
    return int(lib().li_pq_workspace_bytes(B, S, H, m, k))


def pq_search_rerank(q, w, codebook, sigma, codes, k_full, m, k, nv=None, want_shortlist=True, workspace=None,
                     out=None):
    """Two-stage search over product-quantised keys.  q [B, H, 128] bf16, w [B, H],
    codebook [32, 256, 4] int8 (scale sigma), codes [B, S, 32] uint8, k_full
    [B, S, 128] bf16 -> (shortlist [B, m] or None, idx [B, k], val [B, k] fp64)."""
    for t, n in ((q, "q"), (w, "w"), (codebook, "codebook"), (codes, "codes"), (k_full, "k_full")):
        _dev(t, n)
    B, H, d = q.shape
    S = codes.shape[1]
    if out is None:
        sl = torch.empty((B, m), dtype=torch.int32, device=q.device) if want_shortlist else None
        idx = torch.empty((B, k), dtype=torch.int32, device=q.device)
        val = torch.empty((B, k), dtype=torch.float64, device=q.device)
    else:
        sl, idx, val = out
    ws, nb = _workspace(pq_workspace_bytes(B, S, H, m, k), q.device, workspace)
    st = lib().li_pq_search_rerank(_ptr(q), _ptr(w), _ptr(codebook), float(sigma), _ptr(codes), _ptr(k_full),
                                   _ptr(nv), B, S, H, d, m, k, _ptr(sl), _ptr(idx), _ptr(val), _ptr(ws), nb,
                                   _stream(q.device))
    _check(st, "li_pq_search_rerank")
    return sl, idx, val


def sparse_attn_gather(q, kv, idx, sm_scale, with_lse=True, workspace=None, out=None):
    """q [B, Hq, 576] bf16, kv [B, S, 576] bf16, idx [B, k] int32 ->
    (out [B, Hq, 512] bf16, lse [B, Hq] fp32 or None)."""
    _dev(q, "q"); _dev(kv, "kv"); _dev(idx, "idx")
    B, Hq, dqk = q.shape
    S = kv.shape[1]
    k = idx.shape[1]
    dv = 512
    if out is None:
        o = torch.empty((B, Hq, dv), dtype=torch.bfloat16, device=q.device)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if with_lse else None
    else:
        o, lse = out
    ws, nb = _workspace(lib().li_sparse_attn_workspace_bytes(B, Hq, k, dv), q.device, workspace)
    st = lib().li_sparse_attn_gather(_ptr(q), _ptr(kv), _ptr(idx), B, Hq, S, k, dqk, dv, float(sm_scale), _ptr(o),
                                     _ptr(lse), _ptr(ws), nb, _stream(q.device))
    _check(st, "li_sparse_attn_gather")
    return o, lse


PAGE = 64  # keys per page of the paged indexer key cache


def indexer_score_paged(q, w, k_pool, k_scale_pool, page_table, S, nv=None, out=None):
    """Scores [B*T, S] of q [B, T, H, 128] (bf16), w [B, T, H] over a paged fp8 key
    cache: k_pool [num_pages, 64, 128] float8_e4m3fn, k_scale_pool [num_pages, 64],
    page_table [B, max_pages] int32 (pool page of keys 64 p .. 64 p + 63)."""
    for t, n in ((q, "q"), (w, "w"), (k_pool, "k_pool"), (k_scale_pool, "k_scale_pool"), (page_table, "page_table")):
        _dev(t, n)
    B, T, H, d = q.shape
    num_pages = k_pool.shape[0]
    max_pages = page_table.shape[1]
    if out is None:
        out = torch.empty((B * T, S), dtype=torch.float32, device=q.device)
    st = lib().li_indexer_score_paged(_ptr(q), _dtype_code(q, "q"), _ptr(w), _ptr(k_pool), _ptr(k_scale_pool),
                                      _ptr(page_table), PAGE, max_pages, num_pages, _ptr(nv), B, T, S, H, d,
                                      _ptr(out), _stream(q.device))
    _check(st, "li_indexer_score_paged")
    return out


def indexer_topk_paged_workspace_bytes(B, T, S, H, topk):
    return int(lib().li_indexer_topk_paged_workspace_bytes(B, T, S, H, topk))


def indexer_topk_paged(q, w, k_pool, k_scale_pool, page_table, S, topk, nv=None, with_values=True, workspace=None,
                       out=None):
    """(idx [B*T, topk], val [B*T, topk] or None) over a paged fp8 key cache (see
    indexer_score_paged)."""
    for t, n in ((q, "q"), (w, "w"), (k_pool, "k_pool"), (k_scale_pool, "k_scale_pool"), (page_table, "page_table")):
        _dev(t, n)
    B, T, H, d = q.shape
    R = B * T
    if out is None:
        idx = torch.empty((R, topk), dtype=torch.int32, device=q.device)
        val = torch.empty((R, topk), dtype=torch.float32, device=q.device) if with_values else None
    else:
        idx, val = out
    ws, nb = _workspace(indexer_topk_paged_workspace_bytes(B, T, S, H, topk), q.device, workspace)
    st = lib().li_indexer_topk_paged(_ptr(q), _dtype_code(q, "q"), _ptr(w), _ptr(k_pool), _ptr(k_scale_pool),
                                     _ptr(page_table), PAGE, page_table.shape[1], k_pool.shape[0], _ptr(nv), B, T, S,
                                     H, d, topk, _ptr(idx), _ptr(val), _ptr(ws), nb, _stream(q.device))
    _check(st, "li_indexer_topk_paged")
    return idx, val


def sparse_attn_gather_paged(q, kv_pool, slot_table, S, idx, sm_scale, with_lse=True, out=None):
    """q [B, Hq, 576] bf16, kv_pool [num_slots, 576] bf16, slot_table [B, max_slots]
    int32 (pool row of token s of b), idx [B, k] -> (out [B, Hq, 512], lse)."""
    for t, n in ((q, "q"), (kv_pool, "kv_pool"), (slot_table, "slot_table"), (idx, "idx")):
        _dev(t, n)
    B, Hq, dqk = q.shape
    k = idx.shape[1]
    dv = 512
    if out is None:
        o = torch.empty((B, Hq, dv), dtype=torch.bfloat16, device=q.device)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if with_lse else None
    else:
        o, lse = out
    st = lib().li_sparse_attn_gather_paged(_ptr(q), _ptr(kv_pool), _ptr(slot_table), slot_table.shape[1],
                                           kv_pool.shape[0], _ptr(idx), B, Hq, S, k, dqk, dv, float(sm_scale),
                                           _ptr(o), _ptr(lse), _stream(q.device))
    _check(st, "li_sparse_attn_gather_paged")
    return o, lse


def layer_stream_buffer_bytes(S, kv_row_bytes):
    return int(lib().li_layer_stream_buffer_bytes(S, kv_row_bytes))


def layer_stream_prefill(q, w, host_keys, topk, nv=None, host_kv=None, new_rows=0, host_new_keys=None,
                         host_new_kv=None, bufs=None, idx=None, compute=None, copy=None, events=None):
    """Streams L layers of history through two device buffers while each layer's
    chunk is scored and selected (li_layer_stream_prefill).  q [L, T, H, 128] bf16 and
    w [L, T, H] on the device; host_keys [L, S, 128] bf16 and host_kv [L, S, kv_row]
    uint8 in pinned host memory; returns idx [L, T, topk].  compute and copy are
    torch streams (default: the current stream and a new one); events four
    torch.cuda.Event objects (created here if None)."""
    _dev(q, "q"); _dev(w, "w")
    for t, n in ((host_keys, "host_keys"), (host_kv, "host_kv"), (host_new_keys, "host_new_keys"),
                 (host_new_kv, "host_new_kv")):
        if t is not None and not (isinstance(t, torch.Tensor) and not t.is_cuda and t.is_pinned()
                                  and t.is_contiguous()):
            raise TypeError(f"{n} must be a contiguous pinned host tensor")
    L, T, H, d = q.shape
    S = host_keys.shape[1]
    kv_row = host_kv.shape[2] if host_kv is not None else 0
    nb = layer_stream_buffer_bytes(S, kv_row)
    if bufs is None:
        bufs = [torch.empty(nb, dtype=torch.uint8, device=q.device) for _ in range(2)]
    if idx is None:
        idx = torch.empty((L, T, topk), dtype=torch.int32, device=q.device)
    compute = compute or torch.cuda.current_stream(q.device)
    copy = copy or torch.cuda.Stream(device=q.device)
    if events is None:
        events = [torch.cuda.Event() for _ in range(4)]
    for e in events:  # the raw event exists once recorded
        e.record(compute)
    evs = (ctypes.c_void_p * 4)(*[e.cuda_event for e in events])
    st = lib().li_layer_stream_prefill(_ptr(q), _ptr(w), _ptr(nv), _ptr(host_keys), _ptr(host_kv), kv_row,
                                       _ptr(host_new_keys), _ptr(host_new_kv), new_rows, _ptr(bufs[0]), _ptr(bufs[1]),
                                       min(b.numel() for b in bufs), L, T, S, H, d, topk, _ptr(idx),
                                       ctypes.c_void_p(compute.cuda_stream), ctypes.c_void_p(copy.cuda_stream), evs)
    _check(st, "li_layer_stream_prefill")
    return idx

