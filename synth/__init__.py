"""Seeded synthetic inputs shared by the checker and the GPU path.

Only random draws and storage-format encodings live here (see gen.c); nothing in
this package scores, selects or attends.  Every tensor is a pure function of
(seed, tensor id, flat index), so any row can be rebuilt alone.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_u64 = ctypes.c_uint64
_dbl = ctypes.c_double
_ptr = ctypes.c_void_p


def lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "libsynth.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(path)
        for name in ("synth_normal_f64", "synth_normal_f32", "synth_normal_bf16"):
            getattr(L, name).argtypes = [_u64, _u64, _u64, _u64, _dbl, _ptr]
            getattr(L, name).restype = None
        for name in ("synth_uniform_f32", "synth_uniform_f64"):
            getattr(L, name).argtypes = [_u64, _u64, _u64, _u64, _dbl, _dbl, _ptr]
            getattr(L, name).restype = None
        L.synth_normal_bf16_rows.argtypes = [_u64, _u64, _ptr, _u64, _u64, _dbl, _ptr]
        L.synth_normal_bf16_rows.restype = None
        L.synth_fp8_rows.argtypes = [_u64, _u64, _u64, _u64, _u64, _dbl, _ptr, _ptr]
        L.synth_fp8_rows.restype = None
        L.synth_compact_keys.argtypes = [_ptr, _u64, _u64, _ptr, _u64, _ptr, _ptr]
        L.synth_compact_keys.restype = None
        L.synth_pq_codebook.argtypes = [_ptr, _u64, _u64, _u64, ctypes.c_int, _ptr, _ptr]
        L.synth_pq_codebook.restype = None
        L.synth_pq_encode.argtypes = [_ptr, _u64, _u64, _ptr, ctypes.c_float, _ptr]
        L.synth_pq_encode.restype = None
        L.synth_bf16_rne.argtypes = [_dbl]
        L.synth_bf16_rne.restype = ctypes.c_uint16
        L.synth_e4m3_rne.argtypes = [_dbl]
        L.synth_e4m3_rne.restype = ctypes.c_uint8
        L.synth_stream_base.argtypes = [_u64, _u64]
        L.synth_stream_base.restype = _u64
        L.synth_threads.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _n(shape):
    return int(np.prod(shape, dtype=np.int64))


def normal_f64(seed, tid, shape, scale=1.0, off=0):
    out = np.empty(shape, np.float64)
    lib().synth_normal_f64(seed, tid, off, _n(shape), scale, _p(out))
    return out


def normal_f32(seed, tid, shape, scale=1.0, off=0):
    out = np.empty(shape, np.float32)
    lib().synth_normal_f32(seed, tid, off, _n(shape), scale, _p(out))
    return out


def normal_bf16(seed, tid, shape, scale=1.0, off=0, out=None):
    """bf16 bit patterns (uint16) of scale * N(0,1), rounded to nearest even."""
    if out is None:
        out = np.empty(shape, np.uint16)
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.size == _n(shape)
    lib().synth_normal_bf16(seed, tid, off, _n(shape), scale, _p(out))
    return out


def normal_bf16_rows(seed, tid, rows, d, scale=1.0):
    """Rows `rows` (flat row numbers) of a bf16-normal tensor with row length d."""
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, d), np.uint16)
    lib().synth_normal_bf16_rows(seed, tid, _p(rows), rows.size, d, scale, _p(out))
    return out


def uniform_f32(seed, tid, shape, lo=0.0, hi=1.0, off=0):
    out = np.empty(shape, np.float32)
    lib().synth_uniform_f32(seed, tid, off, _n(shape), lo, hi, _p(out))
    return out


def uniform_f64(seed, tid, shape, lo=0.0, hi=1.0, off=0):
    out = np.empty(shape, np.float64)
    lib().synth_uniform_f64(seed, tid, off, _n(shape), lo, hi, _p(out))
    return out


def fp8_rows(seed, tid, rows, d, scale=1.0, row_off=0, codes=None, scales=None):
    """(codes uint8 [rows, d], scales float32 [rows]): N(0,1)*scale rows stored as
    OCP E4M3FN codes with a per-row fp32 scale (rowmax/448)."""
    if codes is None:
        codes = np.empty((rows, d), np.uint8)
    if scales is None:
        scales = np.empty((rows,), np.float32)
    assert codes.size == rows * d and scales.size == rows
    lib().synth_fp8_rows(seed, tid, row_off, rows, d, scale, _p(codes), _p(scales))
    return codes, scales


def compact_keys(k_bf16, P):
    """int8 compact keys of bf16 keys [rows, d] under projection P [dc, d] (float32)."""
    k_bf16 = np.ascontiguousarray(k_bf16, dtype=np.uint16)
    P = np.ascontiguousarray(P, dtype=np.float32)
    d = k_bf16.shape[-1]
    rows = k_bf16.size // d
    dc = P.shape[0]
    assert P.shape[1] == d
    c = np.empty(k_bf16.shape[:-1] + (dc,), np.int8)
    cs = np.empty(k_bf16.shape[:-1], np.float32)
    lib().synth_compact_keys(_p(k_bf16), rows, d, _p(P), dc, _p(c), _p(cs))
    return c, cs


def pq_codebook(k_bf16, seed, iters=8):
    """(cb int8 [d/4, 256, 4], sigma float): k-means codebooks of the 4-dim pieces of
    bf16 keys [n, d] (Lloyd iterations from seeded sample points), stored as int8
    entries with one scale."""
    k_bf16 = np.ascontiguousarray(k_bf16, dtype=np.uint16)
    d = k_bf16.shape[-1]
    n = k_bf16.size // d
    cb = np.empty((d // 4, 256, 4), np.int8)
    sg = ctypes.c_float(0.0)
    lib().synth_pq_codebook(_p(k_bf16), n, d, seed, iters, _p(cb), ctypes.byref(sg))
    return cb, float(sg.value)


def pq_encode(k_bf16, cb, sigma):
    """Codes uint8 [..., d/4] of bf16 keys [..., d]: the nearest entry of each
    piece's codebook."""
    k_bf16 = np.ascontiguousarray(k_bf16, dtype=np.uint16)
    cb = np.ascontiguousarray(cb, dtype=np.int8)
    d = k_bf16.shape[-1]
    rows = k_bf16.size // d
    codes = np.empty(k_bf16.shape[:-1] + (d // 4,), np.uint8)
    lib().synth_pq_encode(_p(k_bf16), rows, d, _p(cb), sigma, _p(codes))
    return codes


def bf16_rne(x: float) -> int:
    return int(lib().synth_bf16_rne(float(x)))


def e4m3_rne(x: float) -> int:
    return int(lib().synth_e4m3_rne(float(x)))


def threads() -> int:
    return int(lib().synth_threads())
