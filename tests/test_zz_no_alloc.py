"""li_topk_select_noalloc (the selection without a workspace, for callers that
cannot allocate) through the C ABI against li_topk_select with a workspace: equal
indices and values bit for bit, on two calls in a row on the shared static scratch,
the second with a smaller input, then a shape that needs no scratch, then the
first shape again."""
import ctypes

import numpy as np
import pytest
import torch

import lightning_indexer_top_amd as li
import oracle
import synth
from helpers import dev

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 34078720  # LI_TOPK_NOALLOC_SCRATCH_BYTES


def scores_of(seed, R, S):
    s = synth.normal_f32(0x5EED0700 + seed, 1, (R, S))
    s[:, ::97] = np.round(s[:, ::97] * 4) / 4  # some ties
    return s


def noalloc(scores, k, nv=None):
    R, S = scores.shape
    idx = torch.empty((R, k), dtype=torch.int32, device="cuda")
    val = torch.empty((R, k), dtype=torch.float32, device="cuda")
    st = li.lib().li_topk_select_noalloc(ctypes.c_void_p(scores.data_ptr()),
                                         None if nv is None else ctypes.c_void_p(nv.data_ptr()), R, S, k,
                                         ctypes.c_void_p(idx.data_ptr()), ctypes.c_void_p(val.data_ptr()),
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, li.lib().li_last_error()
    return idx, val


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_workspace_entry_point(order):
    cases = [
        (1, 16, 131072, 512, None),                                   # the decode shape: uses the scratch
        (2, 6, 40000, 300, np.array([40000, 0, 299, 300, 301, 20000], np.int32)),  # smaller, ragged
        (3, 200, 1000, 64, None),                                     # one workgroup per row: no scratch
        (1, 16, 131072, 512, None),                                   # the first shape again
    ]
    for seed, R, S, k, nv in cases:
        print("noalloc topk", R, S, k, nv is not None, flush=True)
        assert li.topk_workspace_bytes(R, S, k) <= SCRATCH_BYTES
        s = scores_of(seed, R, S)
        ds = dev(s)
        dnv = dev(nv) if nv is not None else None
        i1, v1 = noalloc(ds, k, dnv)
        i2, v2 = li.topk_select(ds, k, dnv)
        torch.cuda.synchronize()
        assert torch.equal(i1, i2), f"R={R} S={S}: indices differ from the workspace entry point"
        assert torch.equal(v1, v2), f"R={R} S={S}: values differ from the workspace entry point"
        o_idx, o_val = oracle.topk(s.astype(np.float64), k, nv)
        assert np.array_equal(i1.cpu().numpy(), o_idx)
        fin = o_idx >= 0
        assert np.array_equal(v1.cpu().numpy().astype(np.float64)[fin], o_val[fin])
