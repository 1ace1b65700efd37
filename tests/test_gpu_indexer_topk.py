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
