"""The tiny decode step (li_indexer_score + li_topk_select, fp32, one row of 4,096
keys, top-64) captured in a HIP graph: every replay, with new inputs copied in and
eager work and synchronisations between replays, equals the same calls run
eagerly, bit for bit.  Neither call records a memset into the graph (the top-k of
a 4,096-key row needs no workspace; the scoring kernel writes every score)."""
import ctypes

import numpy as np
import pytest
import torch

import lightning_indexer_top_amd as li
from synth import workloads
from helpers import dev

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def test_tiny_decode_graph_replays():
    print("graph replays", flush=True)
    sp = workloads.spec("tiny_decode")
    B, S, H, k = sp["B"], sp["S"], sp["H"], sp["topk"]
    L = li.lib()
    assert L.li_topk_workspace_bytes(B, S, k) == 0
    x0 = workloads.indexer_inputs(workloads.spec("tiny_decode", seed=0x5EED1400))
    q, w, kk = dev(x0["q"]).clone(), dev(x0["w"]).clone(), dev(x0["k"]).clone()
    scores = torch.empty((B, S), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    val = torch.empty((B, k), dtype=torch.float32, device="cuda")

    def calls(stream):
        st = ctypes.c_void_p(stream.cuda_stream)
        s = L.li_indexer_score(_p(q), li.LI_F32, _p(w), _p(kk), li.LI_F32, None, None, B, 1, S, H, 128, _p(scores),
                               st)
        s |= L.li_topk_select(_p(scores), None, B, S, k, _p(idx), _p(val), None, ctypes.c_size_t(0), st)
        assert s == 0, L.li_last_error().decode()

    def load(seed):
        x = workloads.indexer_inputs(workloads.spec("tiny_decode", seed=seed))
        q.copy_(dev(x["q"]))
        w.copy_(dev(x["w"]))
        kk.copy_(dev(x["k"]))

    calls(torch.cuda.current_stream())  # one eager call first (kernel attributes set outside capture)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            calls(side)
    torch.cuda.synchronize()
    for rep in range(5):
        load(0x5EED1401 + rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        gi, gv, gs = idx.clone(), val.clone(), scores.clone()
        scores.fill_(float("nan"))  # eager work between replays
        calls(torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert torch.equal(gs, scores), f"replay {rep}: scores"
        assert torch.equal(gi, idx) and torch.equal(gv, val), f"replay {rep}: selection"
        assert (gi >= 0).all() and (gi < S).all()
