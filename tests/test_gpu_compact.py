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
    x = workloads.compact_inputs(sp)
    sl, idx, val = li.compact_search_rerank(dev(x["q"], "bf16"), dev(x["w"]), dev(x["P"]), dev(x["c"]), dev(x["cs"]),
                                            dev(x["k_full"], "bf16"), m, k, dev(nv) if nv is not None else None)
    torch.cuda.synchronize()
    ref = oracle.compact_search(x["q"], x["w"], x["P"], x["c"], x["cs"], x["k_full"], m, k, nv)
    return sl.cpu().numpy(), idx.cpu().numpy(), val.cpu().numpy(), ref


@pytest.mark.parametrize("B,S,H,m,k", [(3, 5000, 64, 2048, 512), (2, 3001, 64, 256, 64), (2, 700, 16, 128, 128),
                                       (1, 2048, 128, 2048, 2048)])
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
