"""End-to-end selection (li_indexer_topk) against the fp64 oracle: index sets equal
up to keys whose oracle score is within 1e-3 relative of the k-th score, and the
GPU's selection equal to the oracle's selection of the GPU's own scores."""
import numpy as np
import pytest
import torch

import lightning_indexer_top_amd as li
import oracle
from synth import workloads
from helpers import assert_topk_band, dev, key_kind, q_kind

pytestmark = pytest.mark.gpu

OT = {"f32": oracle.F32, "bf16": oracle.BF16, "fp8": oracle.FP8_E4M3}
KT = {"f32": li.LI_F32, "bf16": li.LI_BF16, "fp8": li.LI_FP8_E4M3}


def inputs(sp):
    x = workloads.indexer_inputs(sp)
    d = dict(q=dev(x["q"], q_kind(sp)), w=dev(x["w"]), k=dev(x["k"], key_kind(sp)),
             k_scale=dev(x["k_scale"]) if x["k_scale"] is not None else None,
             nv=dev(x["nv"]) if x["nv"] is not None else None)
    return x, d


@pytest.mark.parametrize("name,over", [
    ("tiny_decode", {}),
    ("batched_decode", dict(B=3, S=20000)),
    ("prefill_chunk", dict(T=32, S=4096)),
    ("select_attend", dict(B=2, S=9000)),
])
def test_selection_matches_oracle(name, over):
    print("indexer_topk", name, over, flush=True)
    sp = workloads.spec(name, **over)
    x, d = inputs(sp)
    k = sp["topk"]
    g_idx, g_val = li.indexer_topk(d["q"], d["w"], d["k"], k, d["k_scale"], d["nv"])
    g_scores = li.indexer_score(d["q"], d["w"], d["k"], d["k_scale"], d["nv"])
    torch.cuda.synchronize()
    g_idx = g_idx.cpu().numpy()
    o = oracle.indexer_score(x["q"], OT[sp["q"]], x["w"], x["k"], OT[sp["key"]], x["k_scale"], x["nv"])
    assert_topk_band(g_idx, o, k, x["nv"], name)
    # same precision decision: the oracle's selection of the GPU's own fp32 scores
    gs = g_scores.cpu().numpy().astype(np.float64)
    r_idx, r_val = oracle.topk(gs, k, x["nv"])
    assert np.array_equal(g_idx, r_idx)
    fin = r_idx >= 0
    assert np.array_equal(g_val.cpu().numpy().astype(np.float64)[fin], r_val[fin])


def _fused_check(x, sp, k, what):
    d = dict(q=dev(x["q"], "bf16"), w=dev(x["w"]), k=dev(x["k"], "bf16"),
             nv=dev(x["nv"]) if x["nv"] is not None else None)
    B, T, H = x["q"].shape[:3]
    S = x["k"].shape[1]
    # the fused many-row path needs no workspace: a call with none at all
    assert li.indexer_topk_workspace_bytes(li.LI_BF16, li.LI_BF16, B, T, S, H, k) == 0
    g_idx = torch.empty((B * T, k), dtype=torch.int32, device="cuda")
    g_val = torch.empty((B * T, k), dtype=torch.float32, device="cuda")
    st = li.lib().li_indexer_topk(d["q"].data_ptr(), li.LI_BF16, d["w"].data_ptr(), d["k"].data_ptr(), li.LI_BF16,
                                  None, None if d["nv"] is None else d["nv"].data_ptr(), B, T, S, H, 128, k,
                                  g_idx.data_ptr(), g_val.data_ptr(), None, 0,
                                  torch.cuda.current_stream().cuda_stream)
    assert st == 0, li.lib().li_last_error()
    g_scores = li.indexer_score(d["q"], d["w"], d["k"], None, d["nv"])
    torch.cuda.synchronize()
    g_idx = g_idx.cpu().numpy()
    gs = g_scores.cpu().numpy().astype(np.float64)
    r_idx, r_val = oracle.topk(gs, k, x["nv"])
    assert np.array_equal(g_idx, r_idx), what
    fin = r_idx >= 0
    assert np.array_equal(g_val.cpu().numpy().astype(np.float64)[fin], r_val[fin]), what
    o = oracle.indexer_score(x["q"], oracle.BF16, x["w"], x["k"], oracle.BF16, None, x["nv"])
    assert_topk_band(g_idx, o, k, x["nv"], what)


@pytest.mark.parametrize("T,S,H,k", [(100, 20000, 64, 512), (16, 5000, 8, 64), (40, 3000, 100, 200),
                                     (24, 1500, 32, 512), (16, 70000, 64, 512)])
def test_fused_prefill_shapes(T, S, H, k):
    # query rows scored and selected in one kernel (the scores are never written)
    print("fused prefill", T, S, H, k, flush=True)
    sp = workloads.spec("prefill_chunk", T=T, S=S, H=H, seed=0x5EED0B00 + T + S)
    x = workloads.indexer_inputs(sp)
    _fused_check(x, sp, k, f"T={T} S={S} H={H} k={k}")


@pytest.mark.parametrize("T,S,H,k", [(100, 20000, 64, 512), (16, 5000, 8, 64), (40, 3000, 100, 200)])
def test_fused_prefill_fp8_keys(T, S, H, k):
    # fp8 keys through the fused prefill kernel: no workspace, the selection of the
    # GPU's own (scaled) scores, and the oracle band
    print("fused prefill fp8", T, S, H, k, flush=True)
    sp = workloads.spec("prefill_chunk", T=T, S=S, H=H, key="fp8", seed=0x5EED0E00 + T + S)
    x, d = inputs(sp)
    B = 1
    assert li.indexer_topk_workspace_bytes(li.LI_BF16, li.LI_FP8_E4M3, B, T, S, H, k) == 0
    g_idx = torch.empty((B * T, k), dtype=torch.int32, device="cuda")
    g_val = torch.empty((B * T, k), dtype=torch.float32, device="cuda")
    st = li.lib().li_indexer_topk(d["q"].data_ptr(), li.LI_BF16, d["w"].data_ptr(), d["k"].data_ptr(),
                                  li.LI_FP8_E4M3, d["k_scale"].data_ptr(), d["nv"].data_ptr(), B, T, S, H, 128, k,
                                  g_idx.data_ptr(), g_val.data_ptr(), None, 0,
                                  torch.cuda.current_stream().cuda_stream)
    assert st == 0, li.lib().li_last_error()
    g_scores = li.indexer_score(d["q"], d["w"], d["k"], d["k_scale"], d["nv"])
    torch.cuda.synchronize()
    g_idx = g_idx.cpu().numpy()
    r_idx, r_val = oracle.topk(g_scores.cpu().numpy().astype(np.float64), k, x["nv"])
    assert np.array_equal(g_idx, r_idx)
    fin = r_idx >= 0
    assert np.array_equal(g_val.cpu().numpy().astype(np.float64)[fin], r_val[fin])
    o = oracle.indexer_score(x["q"], oracle.BF16, x["w"], x["k"], oracle.FP8_E4M3, x["k_scale"], x["nv"])
    assert_topk_band(g_idx, o, k, x["nv"], f"fp8 T={T} S={S} H={H} k={k}")


def test_fused_prefill_ties_and_masks():
    # integer-valued queries and keys: many exactly equal scores, so the list
    # compactions resolve ties by index; visible counts 0, below k, at k, ragged
    print("fused prefill ties", flush=True)
    rng = np.random.default_rng(7)
    T, S, H, k = 32, 9000, 64, 512
    import synth
    qf = rng.integers(-2, 3, (1, T, H, 128)).astype(np.float64)
    kf = rng.integers(-1, 2, (1, S, 128)).astype(np.float64)
    q = np.array([synth.bf16_rne(v) for v in qf.ravel()], np.uint16).reshape(qf.shape)
    kk = np.array([synth.bf16_rne(v) for v in kf.ravel()], np.uint16).reshape(kf.shape)
    w = rng.integers(0, 3, (1, T, H)).astype(np.float32)
    nv = rng.integers(600, S + 1, T).astype(np.int32)
    nv[:5] = [0, 1, 511, 512, 513]
    x = {"q": q, "w": w, "k": kk, "nv": nv}
    _fused_check(x, None, k, "ties")


def _a256(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("over,topk,nvs", [
    (dict(B=6, S=131072), 512, None),
    (dict(B=8, S=131072, H=8, key="bf16"), 512, None),
    (dict(B=4, S=70001, H=100), 512, None),
    (dict(B=6, S=140000), 512, [140000, 0, 300, 513, 139999, 70000]),
    (dict(B=8, S=131072, H=32), 2048, None),
    (dict(B=5, S=100000, H=8), 512, [100000, 12345, 0, 600, 99999]),
    (dict(B=6, S=131072), 1, None),
])
def test_decode_select_fused(over, topk, nvs):
    """Few long rows: li_indexer_topk lists every region's entries above a threshold
    of the region's own (inside the scoring kernel for fp8 keys at up to 64 heads,
    after it otherwise) and one finalize selects.  The result must equal
    score-then-select bit for bit, pass the oracle band on every row, repeat on the
    same workspace, follow other queries on that workspace, and come out the same
    from a workspace of arbitrary bytes."""
    print("decode select fused", over, topk, nvs, flush=True)
    sp = workloads.spec("batched_decode", seed=0x5EED0400 + topk + over["B"], **over)
    x, d = inputs(sp)
    R, S, H = sp["B"], sp["S"], sp["H"]
    nv = None
    if nvs is not None:
        nv = np.asarray(nvs, np.int32)
        d["nv"] = dev(nv)
    nb = li.indexer_topk_workspace_bytes(li.LI_BF16, KT[sp["key"]], R, 1, S, H, topk)
    assert nb == _a256(R * S * 4) + li.lib().li_topk_workspace_bytes(R, S, topk)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    i1, v1 = li.indexer_topk(d["q"], d["w"], d["k"], topk, d["k_scale"], d["nv"], workspace=ws)
    torch.cuda.synchronize()
    check_local_thresholds(ws, R, S, topk, nv, v1, d, sp, x, i1)


def ordk(f):
    """Orderable unsigned image of an fp32 value (larger value, larger image)."""
    u = int(np.float32(f).view(np.uint32))
    return (u | 0x80000000) if u < 0x80000000 else (~u & 0xFFFFFFFF)


def check_local_thresholds(ws, R, S, topk, nv, v1, d, sp, x, i1):
    """Every region of a row listed its entries above a threshold of its own
    (per-region counts and thresholds in the workspace), the
    finalize used the lists (the kth value reaches every threshold) or selected over
    the whole row; either way the result equals score-then-select bit for bit, on
    repeated calls, other queries and a workspace of arbitrary bytes."""
    # after the scores: the threshold area (256 words a row), then the region counts
    off = _a256(R * S * 4)
    tu = ws[off:off + R * 256 * 4].view(torch.int32).cpu().numpy().view(np.uint32).reshape(R, 256)
    n = np.full(R, S) if nv is None else np.minimum(nv, S)
    scores = li.indexer_score(d["q"], d["w"], d["k"], d["k_scale"], d["nv"])
    i4, v4 = li.topk_select(scores, topk, d["nv"])
    torch.cuda.synchronize()
    assert torch.equal(i1, i4) and torch.equal(v1, v4)
    vals = v1.cpu().numpy()
    for r in range(R):
        # words 0..127: the regions' thresholds; 128..255: the largest key of each
        # region (written with at most 128 regions a row), so the largest of them is
        # the row's best score
        if n[r] > 0 and tu[r, 128:].any():
            assert tu[r, 128:].max() == ordk(vals[r].max()), f"row {r}: largest listed key"
        if n[r] >= 64 * topk:
            # a long row of unstructured scores: its best keys spread over the
            # workgroups, so every threshold lies below the kth value and the lists
            # were used
            kth = min(ordk(v) for v in vals[r])
            assert tu[r, :128].max() <= kth, f"row {r}: a region's threshold lies above the kth value"
    # other queries on the same workspace, then a workspace of arbitrary bytes
    qr, wr = d["q"].flip(0).contiguous(), d["w"].flip(0).contiguous()
    i5, v5 = li.indexer_topk(qr, wr, d["k"], topk, d["k_scale"], d["nv"], workspace=ws)
    s5 = li.indexer_score(qr, wr, d["k"], d["k_scale"], d["nv"])
    i6, v6 = li.topk_select(s5, topk, d["nv"])
    ws.fill_(0xA7)
    i3, v3 = li.indexer_topk(d["q"], d["w"], d["k"], topk, d["k_scale"], d["nv"], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(i5, i6) and torch.equal(v5, v6)
    assert torch.equal(i3, i4) and torch.equal(v3, v4)
    o = oracle.indexer_score(x["q"], oracle.BF16, x["w"], x["k"], OT[sp["key"]], x["k_scale"], nv)
    assert_topk_band(i1.cpu().numpy(), o, topk, nv, "fused decode select (local thresholds)")


def test_local_thresholds_concentrated_row():
    """A row whose best keys all sit in one scoring workgroup's range: that
    workgroup's own threshold lies above the row's kth value, so the lists cannot
    be trusted and the finalize selects over the whole row; the result stays exact."""
    print("local thresholds, concentrated row", flush=True)
    sp = workloads.spec("batched_decode", seed=0x5EED0510, B=4, S=131072)
    x = workloads.indexer_inputs(sp)
    ks = x["k_scale"].copy()
    ks[1, 1000:1800] *= 50.0   # row 1: 800 keys far above the rest, inside one workgroup
    ks[2, 5000:5100] *= 50.0   # row 2: 100 of them (below k)
    d = dict(q=dev(x["q"], "bf16"), w=dev(x["w"]), k=dev(x["k"], "fp8"), k_scale=dev(ks))
    R, S, H, topk = sp["B"], sp["S"], sp["H"], 512
    ws = torch.zeros(li.indexer_topk_workspace_bytes(li.LI_BF16, li.LI_FP8_E4M3, R, 1, S, H, topk), dtype=torch.uint8,
                     device="cuda")
    i1, v1 = li.indexer_topk(d["q"], d["w"], d["k"], topk, d["k_scale"], None, workspace=ws)
    scores = li.indexer_score(d["q"], d["w"], d["k"], d["k_scale"])
    i4, v4 = li.topk_select(scores, topk)
    torch.cuda.synchronize()
    assert torch.equal(i1, i4) and torch.equal(v1, v4)
    sel = i1.cpu().numpy()
    assert np.isin(np.arange(1000, 1800), sel[1]).sum() >= 500  # row 1's picks come from the boosted range
    assert np.isin(np.arange(5000, 5100), sel[2]).all()


