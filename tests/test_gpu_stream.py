"""Layer-streamed prefill (li_layer_stream_prefill): every layer's selection equals
li_indexer_topk on that layer's keys, bit for bit (and therefore the oracle's
within the usual rules, checked on sampled rows), and the chunk's new rows come
back to the host byte for byte; L = 1, 2 and more layers, ragged S."""
import numpy as np
import pytest
import torch

import lightning_indexer_top_amd as li
import oracle
from synth import workloads
from helpers import assert_topk_band, dev


def pinned(shape, dtype):
    return torch.empty(shape, dtype=dtype, pin_memory=True)


def run(sp, new_rows):
    L, T, S, H, k, kvr = sp["L"], sp["T"], sp["S"], sp["H"], sp["topk"], sp["kv_row"]
    hk = pinned((L, S, 128), torch.int16)
    hkv = pinned((L, S, kvr), torch.uint8) if kvr else None
    x = workloads.layer_stream_inputs(sp, out_keys=hk.numpy().view(np.uint16),
                                      out_kv=hkv.numpy() if kvr else np.empty((L, S, 0), np.uint8))
    nk = pinned((L, new_rows, 128), torch.int16) if new_rows else None
    nkv = pinned((L, new_rows, kvr), torch.uint8) if new_rows and kvr else None
    q, w, nv = dev(x["q"], "bf16"), dev(x["w"]), dev(x["nv"])
    idx = li.layer_stream_prefill(q, w, hk.view(torch.bfloat16), k, nv, hkv, new_rows, nk, nkv)
    torch.cuda.synchronize()
    return x, idx.cpu().numpy(), nk, nkv


@pytest.mark.gpu
@pytest.mark.parametrize("L,T,S,H,k,kvr,new_rows", [(3, 32, 6007, 64, 64, 576, 8), (1, 16, 3000, 32, 16, 0, 4),
                                                     (2, 64, 20000, 64, 512, 576, 16),
                                                     (5, 48, 9000, 128, 100, 100, 12)])
def test_layers_equal_per_layer_selection(L, T, S, H, k, kvr, new_rows):
    print("layer stream", L, T, S, H, k, kvr, new_rows, flush=True)
    sp = workloads.spec("layer_stream", L=L, T=T, S=S, H=H, topk=k, kv_row=kvr, seed=0x5EED1200 + L + S)
    x, idx, nk, nkv = run(sp, new_rows)
    nvd = dev(x["nv"])
    for l in range(L):
        ref, _ = li.indexer_topk(dev(x["q"][l:l + 1], "bf16"), dev(x["w"][l:l + 1]),
                                 dev(x["keys"][l:l + 1], "bf16"), k, None, nvd, with_values=False)
        torch.cuda.synchronize()
        assert np.array_equal(idx[l], ref.cpu().numpy()), f"layer {l} differs from its own selection"
    # the oracle on sampled rows of the first and last layer
    rows = np.array([0, T // 2, T - 1])
    for l in (0, L - 1):
        o = oracle.indexer_score(x["q"][l:l + 1, rows], oracle.BF16, x["w"][l:l + 1, rows], x["keys"][l:l + 1],
                                 oracle.BF16, None, x["nv"][rows])
        assert_topk_band(idx[l][rows], o, k, x["nv"][rows], f"layer {l}")
    if new_rows:
        assert np.array_equal(nk.numpy().view(np.uint16), x["keys"][:, S - new_rows:])
        if kvr:
            assert np.array_equal(nkv.numpy(), x["kv"][:, S - new_rows:])


@pytest.mark.gpu
def test_layer_stream_full_chunk():
    sp = workloads.spec("layer_stream", L=3)
    print("layer stream full chunk", sp["L"], sp["T"], sp["S"], flush=True)
    x, idx, nk, nkv = run(sp, 1024)
    nvd = dev(x["nv"])
    for l in range(sp["L"]):
        ref, _ = li.indexer_topk(dev(x["q"][l:l + 1], "bf16"), dev(x["w"][l:l + 1]), dev(x["keys"][l:l + 1], "bf16"),
                                 sp["topk"], None, nvd, with_values=False)
        torch.cuda.synchronize()
        assert np.array_equal(idx[l], ref.cpu().numpy()), f"layer {l}"
    assert np.array_equal(nkv.numpy(), x["kv"][:, -1024:])


def test_layer_stream_rejects():
    # validation before anything is enqueued (fake pointers are never touched)
    L_ = li.lib()
    A = 0x10000
    import ctypes
    ev = (ctypes.c_void_p * 4)(A, A, A, A)
    args = dict(q=A, w=A, nv=None, hk=A, hkv=A, kvr=576, nk=None, nkv=None, nr=0, b0=A, b1=A,
                nb=L_.li_layer_stream_buffer_bytes(1000, 576), L=2, T=16, S=1000, H=64, d=128, k=64, idx=A)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return L_.li_layer_stream_prefill(a["q"], a["w"], a["nv"], a["hk"], a["hkv"], a["kvr"], a["nk"], a["nkv"],
                                          a["nr"], a["b0"], a["b1"], a["nb"], a["L"], a["T"], a["S"], a["H"], a["d"],
                                          a["k"], a["idx"], None, None, kw.get("ev", ev))
    assert call(q=None) == 1 and call(hk=None) == 1 and call(hkv=None) == 1 and call(b1=None) == 1
    assert call(ev=(ctypes.c_void_p * 4)(A, A, None, A)) == 1
    assert call(T=8) == 2 and call(k=1024) == 2 and call(d=64) == 2 and call(nr=1001) == 2 and call(L=0) == 2
    assert call(nb=args["nb"] - 1) == 5
    assert call(idx=A + 4) == 4
    assert L_.li_layer_stream_buffer_bytes(1000, 576) == 256000 + 576000
