"""GPU parity of li_pq_search_rerank (product-quantised compact keys): shortlist,
final indices and exact scores bit-identical to the oracle's run of the same
two-stage procedure, at small shapes (every head-tile count, ragged key counts,
visible counts around the shortlist size) and at the full pq_search workload."""
import numpy as np
import pytest
import torch

import lightning_indexer_top_amd as li
import oracle
from synth import workloads
from helpers import dev

pytestmark = pytest.mark.gpu


def run(x, m, k, nv=None):
    sl, idx, val = li.pq_search_rerank(dev(x["q"], "bf16"), dev(x["w"]), dev(x["cb"]), x["sigma"], dev(x["codes"]),
                                       dev(x["k_full"], "bf16"), m, k, dev(nv) if nv is not None else None)
    torch.cuda.synchronize()
    ref = oracle.pq_search(x["q"], x["w"], x["cb"], x["sigma"], x["codes"], x["k_full"], m, k, nv)
    return sl.cpu().numpy(), idx.cpu().numpy(), val.cpu().numpy(), ref


def check(sl, idx, val, ref):
    assert np.array_equal(sl, ref["shortlist"]), "shortlist differs"
    assert np.array_equal(idx, ref["idx"]), "final indices differ"
    fin = ref["idx"] >= 0
    assert np.array_equal(val[fin], ref["val"][fin]), "final values differ"


@pytest.mark.parametrize("B,S,H,m,k", [(3, 5000, 64, 2048, 512), (2, 3001, 64, 256, 64), (2, 700, 16, 128, 128),
                                       (1, 2048, 128, 2048, 2048), (2, 20000, 32, 2048, 512),
                                       (2, 9000, 100, 512, 100)])
def test_bit_exact(B, S, H, m, k):
    print("pq", B, S, H, m, k, flush=True)
    sp = workloads.spec("pq_search", B=B, S=S, H=H, seed=0x5EED1000 + S + H, pq_train_stride=1, pq_iters=4)
    check(*run(workloads.pq_inputs(sp), m, k))


def test_visible_counts():
    print("pq nv", flush=True)
    sp = workloads.spec("pq_search", B=4, S=3000, H=64, seed=0x5EED1100, pq_train_stride=1, pq_iters=4)
    nv = np.array([100, 3000, 2100, 0], np.int32)
    sl, idx, val, ref = run(workloads.pq_inputs(sp), 1024, 256, nv)
    check(sl, idx, val, ref)
    assert (idx[0, 100:] == -1).all() and (idx[3] == -1).all()


def test_pq_search_full_size():
    sp = workloads.spec("pq_search")
    print("full size pq_search", sp["B"], sp["S"], flush=True)
    x = workloads.pq_inputs(sp)
    print("inputs ready; oracle on every sequence", flush=True)
    check(*run(x, sp["m"], sp["topk"]))


def test_multi_region_visible_counts():
    """Rows of at least 16,384 keys: the shortlist comes from per-region lists (fp64
    scores listed on the upper half of the ordered value) and one exact pass, with a
    ragged last region and a visible count inside a region."""
    print("pq multi-region", flush=True)
    sp = workloads.spec("pq_search", B=2, S=40000, H=64, seed=0x5EED1200, pq_train_stride=1, pq_iters=4)
    nv = np.array([40000, 23456], np.int32)
    check(*run(workloads.pq_inputs(sp), 2048, 512, nv))


@pytest.mark.parametrize("H", [64, 32, 128])
def test_stage1_region_lists(H):
    """32 sequences of 131,072 keys: each PQ stage-1 workgroup scores exactly one
    4,096-key region and lists its shortlist candidates itself (its scores read back
    after the workgroup barrier; one, two and four 32-head tiles).  Visible counts
    inside a region, on a region edge, below one region, below the shortlist size
    and zero; every row bit-exact."""
    print("pq stage-1 region lists", H, flush=True)
    sp = workloads.spec("pq_search", H=H, seed=0x5EED1300 + H, pq_iters=2)
    B, S = sp["B"], sp["S"]
    nv = np.full(B, S, np.int32)
    nv[1:6] = [77777, 12288, 4000, 1999, 0]
    sl, idx, val, ref = run(workloads.pq_inputs(sp), sp["m"], sp["topk"], nv)
    check(sl, idx, val, ref)
    assert (idx[5] == -1).all()

