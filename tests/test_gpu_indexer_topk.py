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
    g_idx, g_val = li.indexer_topk(d["q"], d["w"], d["k"], k, None, d["nv"])
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
    (dict(B=6, S=131072), 1, None),
])
def test_decode_select_fused(over, topk, nvs):
    """Few long rows (at least 1,024 keys per scoring workgroup): li_indexer_topk runs
    the scoring kernel with its selection epilogue (threshold from every wave's first
    tile, per-workgroup candidate lists) and one finalize.  The result must equal
    score-then-select bit for bit, pass the oracle band on every row, repeat on the
    same workspace, follow other queries on that workspace, and come out the same
    from a workspace of arbitrary bytes (whose flags send rows through the whole-row
    selection)."""
    print("decode select fused", over, topk, nvs, flush=True)
    sp = workloads.spec("batched_decode", seed=0x5EED0400 + topk + over["B"], **over)
    x, d = inputs(sp)
    R, S, H = sp["B"], sp["S"], sp["H"]
    nv = None
    if nvs is not None:
        nv = np.asarray(nvs, np.int32)
        d["nv"] = dev(nv)
    nb = li.indexer_topk_workspace_bytes(R, 1, S, H, topk)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    i1, v1 = li.indexer_topk(d["q"], d["w"], d["k"], topk, d["k_scale"], d["nv"], workspace=ws)
    torch.cuda.synchronize()
    # every row with more than k visible keys was listed by the scoring kernel: no
    # region is marked unfiltered (regions [R][P], P of them per row), and the
    # finalize cleared the sample flags (1024 words per row after the top-k's area)
    off = _a256(R * S * 4)
    bcnt = ws[off + _a256(R * 8):off + _a256(R * 8) + R * 256 * 4].view(torch.int32).cpu().numpy()
    flags_at = off + _a256(R * 8) + _a256(R * 256 * 4) + 2 * _a256(R * S * 4)
    flags = ws[flags_at:flags_at + R * 1024 * 4].view(torch.int32).cpu().numpy()
    n = np.full(R, S) if nv is None else np.minimum(nv, S)
    regions = bcnt[:R * 256]
    assert (flags == 0).all(), "sample flags not cleared"
    assert (regions != -1).all(), "a region was left unfiltered"
    # the row's threshold was published once (epoch << 32 | threshold, one 128-byte
    # line per row) and every region of the row filtered with it (256 words per row)
    tu_at = flags_at + _a256(R * 1024 * 4)
    pub_at = tu_at + _a256(R * 256 * 4)
    tu = ws[tu_at:tu_at + R * 256 * 4].view(torch.int32).cpu().numpy().view(np.uint32).reshape(R, 256)
    pub = ws[pub_at:pub_at + R * 128].view(torch.int64).cpu().numpy().view(np.uint64).reshape(R, 16)[:, 0]
    for r in range(R):
        if n[r] > topk:
            assert pub[r] >> np.uint64(32) != 0, f"row {r}: no published threshold"
            used = tu[r][tu[r] != 0]
            assert len(used) > 0 and (used == np.uint32(pub[r] & np.uint64(0xFFFFFFFF))).all(), \
                f"row {r}: regions filtered with different thresholds"
    # other queries on the same workspace (rows reversed): every sample comes from
    # this call, nothing from the previous one
    qr, wr = d["q"].flip(0).contiguous(), d["w"].flip(0).contiguous()
    i5, v5 = li.indexer_topk(qr, wr, d["k"], topk, d["k_scale"], d["nv"], workspace=ws)
    torch.cuda.synchronize()
    assert (ws[off + _a256(R * 8):off + _a256(R * 8) + R * 256 * 4].view(torch.int32).cpu().numpy()[:R * 256] != -1).all()
    s5 = li.indexer_score(qr, wr, d["k"], d["k_scale"], d["nv"])
    i6, v6 = li.topk_select(s5, topk, d["nv"])
    assert torch.equal(i5, i6) and torch.equal(v5, v6)
    i2, v2 = li.indexer_topk(d["q"], d["w"], d["k"], topk, d["k_scale"], d["nv"], workspace=ws)
    ws.fill_(0xA7)
    i3, v3 = li.indexer_topk(d["q"], d["w"], d["k"], topk, d["k_scale"], d["nv"], workspace=ws)
    scores = li.indexer_score(d["q"], d["w"], d["k"], d["k_scale"], d["nv"])
    i4, v4 = li.topk_select(scores, topk, d["nv"])
    torch.cuda.synchronize()
    for a, b in ((i1, i4), (i2, i4), (i3, i4)):
        assert torch.equal(a, b)
    for a, b in ((v1, v4), (v2, v4), (v3, v4)):
        assert torch.equal(a, b)
    o = oracle.indexer_score(x["q"], oracle.BF16, x["w"], x["k"], OT[sp["key"]], x["k_scale"], nv)
    assert_topk_band(i1.cpu().numpy(), o, topk, nv, "fused decode select")


@pytest.mark.parametrize("bogus", ["all", "none", "mid"])
def test_decode_select_planted_threshold(bogus):
    """A published threshold word that matches the launch by accident: each fused
    decode launch publishes its rows' thresholds as (epoch << 32 | threshold), the
    epoch counting launches.  Planting the next launch's epoch with a wrong
    threshold in one row's word makes that launch's workgroups filter with it: one
    that keeps every entry (the list overflows), one that keeps none (too short), or
    a plausible one (the lists are used).  The result must equal score-then-select
    bit for bit in every case."""
    print("planted threshold", bogus, flush=True)
    sp = workloads.spec("batched_decode", seed=0x5EED0500, B=8, S=131072)
    x, d = inputs(sp)
    R, S, H, topk = sp["B"], sp["S"], sp["H"], 512
    nb = li.indexer_topk_workspace_bytes(R, 1, S, H, topk)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    li.indexer_topk(d["q"], d["w"], d["k"], topk, d["k_scale"], None, workspace=ws)
    torch.cuda.synchronize()
    off = _a256(R * S * 4)
    flags_at = off + _a256(R * 8) + _a256(R * 256 * 4) + 2 * _a256(R * S * 4)
    pub_at = flags_at + _a256(R * 1024 * 4) + _a256(R * 256 * 4)
    pub = ws[pub_at:pub_at + R * 128].view(torch.int64).cpu().numpy().view(np.uint64).reshape(R, 16)[:, 0]
    epoch = int(pub[0] >> np.uint64(32))
    assert epoch != 0
    scores = li.indexer_score(d["q"], d["w"], d["k"], d["k_scale"])
    i_ref, v_ref = li.topk_select(scores, topk)
    torch.cuda.synchronize()
    row = scores[1].cpu().numpy()
    ordk = lambda f: int(np.float32(f).view(np.uint32) | 0x80000000) if f >= 0 else int(~np.float32(f).view(np.uint32) & 0xFFFFFFFF)
    tau = {"all": 1, "none": 0xFFFFFFFF, "mid": ordk(np.sort(row)[-1500])}[bogus]
    word = np.array([((epoch + 1) << 32) | tau], dtype=np.uint64)
    ws[pub_at + 128:pub_at + 136] = torch.from_numpy(word.view(np.uint8)).cuda()  # row 1
    i1, v1 = li.indexer_topk(d["q"], d["w"], d["k"], topk, d["k_scale"], None, workspace=ws)
    torch.cuda.synchronize()
    pub2 = ws[pub_at:pub_at + R * 128].view(torch.int64).cpu().numpy().view(np.uint64).reshape(R, 16)[:, 0]
    assert int(pub2[0] >> np.uint64(32)) == epoch + 1, "the launch used the planted epoch"
    assert torch.equal(i1, i_ref) and torch.equal(v1, v_ref)
