"""GPU parity of li_compact_search_rerank: shortlist, final indices and exact scores
bit-identical to the oracle's run of the same two-stage procedure."""
import numpy as np
import pytest
import torch

import lightning_indexer_top_amd as li
import oracle
from synth import workloads
from helpers import dev

pytestmark = pytest.mark.gpu


def run(sp, m, k, nv=None):
    return run_x(workloads.compact_inputs(sp), m, k, nv)


def run_x(x, m, k, nv=None):
    sl, idx, val = li.compact_search_rerank(dev(x["q"], "bf16"), dev(x["w"]), dev(x["P"]), dev(x["c"]), dev(x["cs"]),
                                            dev(x["k_full"], "bf16"), m, k, dev(nv) if nv is not None else None)
    torch.cuda.synchronize()
    ref = oracle.compact_search(x["q"], x["w"], x["P"], x["c"], x["cs"], x["k_full"], m, k, nv)
    return sl.cpu().numpy(), idx.cpu().numpy(), val.cpu().numpy(), ref


@pytest.mark.parametrize("B,S,H,m,k", [(3, 5000, 64, 2048, 512), (2, 3001, 64, 256, 64), (2, 700, 16, 128, 128),
                                       (1, 2048, 128, 2048, 2048), (2, 3001, 100, 256, 64), (2, 9000, 48, 512, 100)])
def test_bit_exact(B, S, H, m, k):
    print("compact", B, S, H, m, k, flush=True)
    sp = workloads.spec("compact_search", B=B, S=S, H=H, seed=0x5EED0600 + S)
    sl, idx, val, ref = run(sp, m, k)
    assert np.array_equal(sl, ref["shortlist"])
    assert np.array_equal(idx, ref["idx"])
    fin = ref["idx"] >= 0
    assert np.array_equal(val[fin], ref["val"][fin])


def test_visible_counts():
    print("compact nv", flush=True)
    sp = workloads.spec("compact_search", B=3, S=3000, H=64, seed=0x5EED0700)
    nv = np.array([100, 3000, 2100], np.int32)
    sl, idx, val, ref = run(sp, 1024, 256, nv)
    assert np.array_equal(sl, ref["shortlist"]) and np.array_equal(idx, ref["idx"])
    assert (idx[0, 100:] == -1).all()


def check(sl, idx, val, ref, what):
    assert np.array_equal(sl, ref["shortlist"]), f"{what}: shortlist differs"
    assert np.array_equal(idx, ref["idx"]), f"{what}: final indices differ"
    fin = ref["idx"] >= 0
    assert np.array_equal(val[fin], ref["val"][fin]), f"{what}: final values differ"


def test_multi_region_lists():
    """Rows of at least 16,384 keys take the selection on few long rows: every
    4,096-key region lists its fp64 stage-1 scores above a threshold of its own (on
    the upper half of the ordered value) and one exact pass selects the shortlist.
    A ragged last region, a visible count inside a region, one below the shortlist
    size."""
    print("compact multi-region", flush=True)
    sp = workloads.spec("compact_search", B=3, S=40000, H=64, seed=0x5EED0710)
    nv = np.array([40000, 17000, 1500], np.int32)
    check(*run(sp, 2048, 512, nv), "multi-region")


def test_concentrated_shortlist():
    """Every one of row 0's best stage-1 scores in one 4,096-key region (its
    compact-key scales multiplied by 64): that region's own threshold lies above
    the row's 2,048th value, so its lists cannot be used and the row is selected
    whole; row 1 is left as drawn.  Both bit-exact."""
    print("compact concentrated", flush=True)
    sp = workloads.spec("compact_search", B=2, S=40000, H=64, seed=0x5EED0720)
    x = workloads.compact_inputs(sp)
    x["cs"] = np.array(x["cs"], copy=True)
    x["cs"][0, 4096:8192] *= 64.0
    check(*run_x(x, 2048, 512), "concentrated")


@pytest.mark.parametrize("H", [64, 32, 128])
def test_stage1_region_lists(H):
    """32 sequences of 131,072 keys: each stage-1 workgroup scores exactly one
    4,096-key region and lists its shortlist candidates itself (one, two and four
    32-head tiles).  Visible counts inside a region, on a region edge, below one
    region, below the shortlist size and zero; row 1 has every best score in one
    region (its lists cannot be used, so the row is selected whole).  Every row
    bit-exact."""
    print("compact stage-1 region lists", H, flush=True)
    sp = workloads.spec("compact_search", H=H, seed=0x5EED0730 + H)
    B, S = sp["B"], sp["S"]
    x = workloads.compact_inputs(sp)
    x["cs"] = np.array(x["cs"], copy=True)
    x["cs"][1, 8192:12288] *= 64.0
    nv = np.full(B, S, np.int32)
    nv[2:8] = [100000, 8192, 4096, 3000, 1500, 0]
    nv[9] = 16385
    sl, idx, val, ref = run_x(x, 2048, 512, nv)
    check(sl, idx, val, ref, "stage-1 region lists")
    assert (idx[7] == -1).all() and (idx[6, 1500:] == -1).all()

