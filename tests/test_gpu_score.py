"""GPU parity of li_indexer_score against the fp64 oracle (every element) on small
shapes spanning several key tiles and a ragged tail, all dtype paths, head counts,
causal masks and the degenerate visible-key counts."""
import numpy as np
import pytest
import torch

import lightning_indexer_top_amd as li
import oracle
import synth
from synth import workloads
from helpers import assert_scores_close, dev, key_kind, q_kind

pytestmark = pytest.mark.gpu

OT = {"f32": oracle.F32, "bf16": oracle.BF16, "fp8": oracle.FP8_E4M3}


def run(sp, nv=None):
    x = workloads.indexer_inputs(sp)
    if nv is not None:
        x["nv"] = nv
    q = dev(x["q"], q_kind(sp))
    w = dev(x["w"])
    k = dev(x["k"], key_kind(sp))
    ks = dev(x["k_scale"]) if x["k_scale"] is not None else None
    nvd = dev(x["nv"]) if x["nv"] is not None else None
    g = li.indexer_score(q, w, k, ks, nvd)
    torch.cuda.synchronize()
    o = oracle.indexer_score(x["q"], OT[sp["q"]], x["w"], x["k"], OT[sp["key"]], x["k_scale"], x["nv"])
    return g.cpu().numpy(), o, x


def test_tiny_decode_full():
    print("tiny_decode", flush=True)
    g, o, _ = run(workloads.spec("tiny_decode"))
    assert_scores_close(g, o, "tiny_decode")


@pytest.mark.parametrize("key", ["fp8", "bf16"])
@pytest.mark.parametrize("H", [1, 8, 32, 48, 64, 100, 128])
def test_decode_heads_and_tail(key, H):
    print("decode", key, H, flush=True)
    sp = workloads.spec("batched_decode", B=2, S=3001, H=H, key=key, seed=0x5EED0100 + H)
    g, o, _ = run(sp)
    assert_scores_close(g, o, f"{key} H={H}")


@pytest.mark.parametrize("combo", [("f32", "f32"), ("f32", "fp8"), ("f32", "bf16"), ("bf16", "f32")])
def test_fp32_paths(combo):
    qt, kt = combo
    print("fp32 path", combo, flush=True)
    sp = workloads.spec("tiny_decode", B=2, S=1500, H=12, q=qt, key=kt, seed=0x5EED0200)
    g, o, _ = run(sp)
    assert_scores_close(g, o, str(combo))


def test_prefill_causal_small():
    print("prefill small", flush=True)
    sp = workloads.spec("prefill_chunk", T=64, S=2048, seed=0x5EED0300)
    g, o, x = run(sp)
    assert_scores_close(g, o, "prefill")
    nv = x["nv"]
    for t in range(64):
        assert np.isneginf(g[t, nv[t]:]).all() and np.isfinite(g[t, : nv[t]]).all()


@pytest.mark.parametrize("B,T,S,H", [(2, 17, 1000, 64), (1, 40, 3001, 100), (3, 64, 513, 8)])
def test_prefill_tiled_scores(B, T, S, H):
    # many query rows (bf16): the MFMA-tiled scoring kernel, ragged row counts (rows
    # past T in a workgroup), ragged key tails and per-row visible counts in [0, S]
    print("prefill tiled", B, T, S, H, flush=True)
    sp = workloads.spec("prefill_chunk", B=B, T=T, S=S, H=H, seed=0x5EED0C00 + T + S)
    rng = np.random.default_rng(T + S)
    nv = rng.integers(0, S + 1, B * T).astype(np.int32)
    nv[0], nv[-1] = 0, S
    g, o, _ = run(sp, nv=nv)
    assert_scores_close(g, o, f"prefill tiled B={B} T={T} S={S} H={H}")
    for r in range(B * T):
        assert np.isneginf(g[r, nv[r]:]).all() and np.isfinite(g[r, : nv[r]]).all()


def test_visible_count_edges():
    print("nv edges", flush=True)
    sp = workloads.spec("batched_decode", B=1, T=6, S=700, H=64, seed=0x5EED0400)
    nv = np.array([0, 1, 31, 33, 700, 5000], np.int32)
    g, o, _ = run(sp, nv=nv)  # counts above S clamp to S, as in the oracle
    assert_scores_close(g, o, "nv edges")
    assert np.isneginf(g[0]).all()


def test_scale_commutes_with_relu():
    # the kernel applies the per-key scale after the head sum; scaling every key's
    # scale by 2 must scale every score by exactly 2
    print("scale", flush=True)
    sp = workloads.spec("batched_decode", B=1, S=600, H=64, seed=0x5EED0500)
    x = workloads.indexer_inputs(sp)
    q, w, k = dev(x["q"], "bf16"), dev(x["w"]), dev(x["k"], "fp8")
    a = li.indexer_score(q, w, k, dev(x["k_scale"]))
    b = li.indexer_score(q, w, k, dev(x["k_scale"] * 2))
    torch.cuda.synchronize()
    assert torch.equal(a * 2, b)
