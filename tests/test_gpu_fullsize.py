"""Parity at each workload's full size, in the launch configuration the benchmark
times: every output row is checked for the properties a selection must have, and
sampled rows (or every row, where the oracle is fast enough) against the fp64
oracle with the same acceptance rules as the small-shape tests."""
import math

import numpy as np
import pytest
import torch

import lightning_indexer_top_amd as li
import oracle
from synth import workloads
from helpers import assert_attn_close, assert_scores_close, assert_topk_band, bf16_host, dev

pytestmark = pytest.mark.gpu


def assert_valid_sets(idx, nv, S, k, what):
    """Every row: min(k, nv) distinct indices in [0, nv), ascending, then -1."""
    idx = np.asarray(idx)
    R = idx.shape[0]
    n = np.full(R, S) if nv is None else np.minimum(np.maximum(np.asarray(nv), 0), S)
    take = np.minimum(k, n)
    pos = np.arange(k)[None, :]
    live = pos < take[:, None]
    assert (idx[~live] == -1).all(), f"{what}: padding"
    assert ((idx >= 0) & (idx < n[:, None]))[live].all(), f"{what}: index out of range"
    inc = np.diff(idx, axis=1) > 0
    assert (inc | ~live[:, 1:]).all(), f"{what}: not strictly ascending"


def stratified_rows(T):
    """Rows t with t mod 16 in {0, 3}, and the first and last 8 rows of the chunk."""
    t = np.arange(T)
    keep = (t % 16 == 0) | (t % 16 == 3) | (t < 8) | (t >= T - 8)
    return t[keep]


def test_stratified_rows_cover_both_phases_and_ends():
    rows = stratified_rows(4096)
    assert len(rows) == 512 + 6 + 8  # rows 0 and 3 of the first eight are in the 16-row pattern
    assert {0, 3, 16, 19, 4093, 4095}.issubset(set(rows.tolist()))


def test_batched_decode_full_size():
    sp = workloads.spec("batched_decode")
    B, S, k = sp["B"], sp["S"], sp["topk"]
    print("full size batched_decode", B, S, flush=True)
    x = workloads.indexer_inputs(sp)
    q, w, kk, ks = dev(x["q"], "bf16"), dev(x["w"]), dev(x["k"], "fp8"), dev(x["k_scale"])
    scores = li.indexer_score(q, w, kk, ks)
    idx, val = li.topk_select(scores, k)
    torch.cuda.synchronize()
    g = scores.cpu().numpy()
    g_idx = idx.cpu().numpy()
    assert_valid_sets(g_idx, None, S, k, "batched_decode")
    # every row against the oracle (one thread per row)
    o = oracle.indexer_score(x["q"], oracle.BF16, x["w"], x["k"], oracle.FP8_E4M3, x["k_scale"])
    assert_scores_close(g, o, "batched_decode scores")
    assert_topk_band(g_idx, o, k, None, "batched_decode top-k")
    r_idx, r_val = oracle.topk(g.astype(np.float64), k)
    assert np.array_equal(g_idx, r_idx)
    assert np.array_equal(val.cpu().numpy().astype(np.float64), r_val)


def test_prefill_chunk_full_size():
    sp = workloads.spec("prefill_chunk")
    T, S, H, k = sp["T"], sp["S"], sp["H"], sp["topk"]
    print("full size prefill_chunk", T, S, flush=True)
    x = workloads.indexer_inputs(sp)
    nv = x["nv"]
    q, w, kk, dnv = dev(x["q"], "bf16"), dev(x["w"]), dev(x["k"], "bf16"), dev(nv)
    # the fused call exactly as the benchmark makes it (no values), then with values
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    li.indexer_topk(q, w, kk, k, None, dnv, with_values=False, out=(idx, None))
    idx2, val2 = li.indexer_topk(q, w, kk, k, None, dnv)
    torch.cuda.synchronize()
    g_idx = idx.cpu().numpy()
    assert np.array_equal(g_idx, idx2.cpu().numpy())
    assert_valid_sets(g_idx, nv, S, k, "prefill_chunk")
    # a stratified subset: every 16th row at both ends of its group of four rows that
    # share a visible count (t mod 16 in {0, 3}), plus the first and last 8 rows
    rows = stratified_rows(T)
    print("oracle rows", len(rows), flush=True)
    o = oracle.indexer_score(x["q"][:, rows], oracle.BF16, x["w"][:, rows], x["k"], oracle.BF16, None, nv[rows])
    assert_topk_band(g_idx[rows], o, k, nv[rows], "prefill_chunk top-k")
    # the unfused scoring kernel on the same rows, and the fused selection equal to
    # the oracle's selection of those GPU scores
    sub = li.indexer_score(q[:, rows].contiguous(), w[:, rows].contiguous(), kk, None, dnv[rows].contiguous())
    torch.cuda.synchronize()
    gs = sub.cpu().numpy()
    assert_scores_close(gs, o, "prefill_chunk scores")
    r_idx, r_val = oracle.topk(gs.astype(np.float64), k, nv[rows])
    assert np.array_equal(g_idx[rows], r_idx)
    fin = r_idx >= 0
    assert np.array_equal(val2.cpu().numpy()[rows].astype(np.float64)[fin], r_val[fin])


def test_compact_search_full_size():
    sp = workloads.spec("compact_search")
    B, S, H, m, k = sp["B"], sp["S"], sp["H"], sp["m"], sp["topk"]
    print("full size compact_search", B, S, flush=True)
    x = workloads.compact_inputs(sp)
    sl, idx, val = li.compact_search_rerank(dev(x["q"], "bf16"), dev(x["w"]), dev(x["P"]), dev(x["c"]),
                                            dev(x["cs"]), dev(x["k_full"], "bf16"), m, k)
    torch.cuda.synchronize()
    sl, idx, val = sl.cpu().numpy(), idx.cpu().numpy(), val.cpu().numpy()
    assert_valid_sets(sl, None, S, m, "shortlist")
    assert_valid_sets(idx, None, S, k, "final")
    assert all(np.isin(idx[b], sl[b]).all() for b in range(B))
    # every sequence, bit for bit
    print("oracle, all", B, "sequences", flush=True)
    o = oracle.compact_search(x["q"], x["w"], x["P"], x["c"], x["cs"], x["k_full"], m, k)
    for b in range(B):
        assert np.array_equal(sl[b], o["shortlist"][b]), f"sequence {b}: shortlist"
        assert np.array_equal(idx[b], o["idx"][b]), f"sequence {b}: final indices"
        assert np.array_equal(val[b], o["val"][b]), f"sequence {b}: final values"


def test_select_attend_full_size():
    sp = workloads.spec("select_attend")
    B, S, k, Hq = sp["B"], sp["S"], sp["topk"], sp["Hq"]
    print("full size select_attend indexer", B, S, flush=True)
    x = workloads.indexer_inputs(sp)
    q, w, kk, ks = dev(x["q"], "bf16"), dev(x["w"]), dev(x["k"], "fp8"), dev(x["k_scale"])
    scores = li.indexer_score(q, w, kk, ks)
    idx, _ = li.topk_select(scores, k, with_values=False)
    torch.cuda.synchronize()
    g_idx = idx.cpu().numpy()
    assert_valid_sets(g_idx, None, S, k, "select_attend")
    g = scores.cpu().numpy()
    r_idx, _ = oracle.topk(g.astype(np.float64), k)
    assert np.array_equal(g_idx, r_idx)
    # every row against the oracle, in four batches of 16 sequences
    for b0 in range(0, B, 16):
        rows = list(range(b0, b0 + 16))
        print("oracle rows", rows[0], "-", rows[-1], flush=True)
        o = oracle.indexer_score(x["q"][rows], oracle.BF16, x["w"][rows], x["k"][rows], oracle.FP8_E4M3,
                                 x["k_scale"][rows])
        assert_scores_close(g[rows], o, "select_attend scores")
        assert_topk_band(g_idx[rows], o, k, None, "select_attend top-k")
        del o
    del scores, kk, ks, x
    torch.cuda.empty_cache()
    # attention over the GPU's own selection, every sequence: the latent cache is
    # allocated at full size and only the selected rows are written
    print("full size select_attend attention", B, Hq, flush=True)
    lat = torch.empty((B, S, sp["dqk"]), dtype=torch.bfloat16, device="cuda")
    rows_h = workloads.latent_rows(sp, g_idx)
    rows_d = dev(rows_h, "bf16")
    for b in range(B):
        lat[b, idx[b].long()] = rows_d[b]
    qa_h = workloads.attn_query(sp)
    out, lse = li.sparse_attn_gather(dev(qa_h, "bf16"), lat, idx, sp["tau"])
    torch.cuda.synchronize()
    o_out, o_lse = oracle.sparse_attn_rows(qa_h, rows_h, g_idx, sp["dv"], sp["tau"])
    assert_attn_close(bf16_host(out), o_out, "select_attend attention")
    np.testing.assert_allclose(lse.cpu().numpy(), o_lse, rtol=1e-3, atol=1e-3)
    del lat
    torch.cuda.empty_cache()
