"""Shared helpers of the GPU parity tests: moving the generators' host arrays to
the device and the acceptance rules of the parity checks."""
import numpy as np
import torch

SCORE_RTOL = 2e-2     # scores, bf16/fp8 inputs: |g - o| <= 2e-2 * max(|o|, 1e-3 * max_row |o|)
BAND_RTOL = 1e-3      # top-k: set differences only inside 1e-3 relative of the k-th score
ATTN_RTOL = 1e-2      # attention: per (b, head) max|g - o| / max|o|


def dev(a, kind=None):
    """numpy host array -> torch device tensor; kind names the storage format."""
    a = np.ascontiguousarray(a)
    if kind == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    if kind == "fp8":
        return torch.from_numpy(a).view(torch.float8_e4m3fn).cuda()
    return torch.from_numpy(a).cuda()


def key_kind(spec):
    return {"f32": None, "bf16": "bf16", "fp8": "fp8"}[spec["key"]]


def q_kind(spec):
    return "bf16" if spec["q"] == "bf16" else None


def bf16_host(t):
    """bf16 device tensor -> float64 numpy array."""
    return t.float().cpu().numpy().astype(np.float64)


def assert_scores_close(g, o, what=""):
    """g: fp32 GPU scores, o: fp64 oracle scores, same shape [R, S]."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    assert g.shape == o.shape
    neg = np.isneginf(o)
    assert np.array_equal(np.isneginf(g), neg), f"{what}: masked positions differ"
    fin = np.where(neg, 0.0, o)
    rowmax = np.abs(fin).max(axis=-1, keepdims=True)
    tol = SCORE_RTOL * np.maximum(np.abs(fin), 1e-3 * rowmax)
    err = np.abs(np.where(neg, 0.0, g) - fin)
    bad = err > tol
    assert not bad.any(), f"{what}: {bad.sum()} scores out of tolerance, worst {err.max():.3e}"


def assert_topk_band(g_idx, o_scores, k, nv=None, what=""):
    """GPU top-k index rows g_idx [R, k] against oracle fp64 scores [R, S]: the sets
    may differ only in keys whose oracle score lies within BAND_RTOL of the k-th."""
    g_idx = np.asarray(g_idx)
    R, S = o_scores.shape
    for r in range(R):
        n = S if nv is None else int(min(max(nv[r], 0), S))
        take = min(k, n)
        row = g_idx[r]
        assert (row[take:] == -1).all(), f"{what} row {r}: padding"
        sel = row[:take]
        assert len(np.unique(sel)) == take, f"{what} row {r}: duplicates"
        assert sel.min(initial=0) >= 0 and sel.max(initial=-1) < n, f"{what} row {r}: out of range"
        if take == 0:
            continue
        o = o_scores[r, :n]
        order = np.lexsort((np.arange(n), -o))
        ref = order[:take]
        sk = o[ref[-1]]
        diff = np.setxor1d(sel, ref)
        if diff.size:
            far = np.abs(o[diff] - sk) > BAND_RTOL * abs(sk)
            assert not far.any(), f"{what} row {r}: {far.sum()} keys outside the near-tie band"


def assert_attn_close(g, o, what=""):
    """g, o: [B, Hq, dv]; per (b, head) max|g - o| / max|o| <= ATTN_RTOL."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    err = np.abs(g - o).max(axis=-1)
    ref = np.abs(o).max(axis=-1)
    rel = err / np.maximum(ref, 1e-30)
    bad = (rel > ATTN_RTOL) & (ref > 0)
    assert not bad.any(), f"{what}: {bad.sum()} rows out of tolerance, worst {rel.max():.3e}"
    assert np.all(g[ref == 0] == 0)
