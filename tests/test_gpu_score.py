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


def test_held_scores_multi_tile_with_visible_ends():
    """fp8 keys at 64 heads on few long rows: on 256 CUs every workgroup streams
    3,072 keys (24 tiles a wave) and holds its scores in LDS until its last tile;
    the visible counts end inside a workgroup, inside a tile and at a workgroup
    edge.  Every element against the oracle."""
    S = 524288
    nv = np.array([S - 777, 300001, 3072 * 51], np.int32)
    print("held scores multi-tile", S, nv.tolist(), flush=True)
    sp = workloads.spec("batched_decode", B=3, S=S, H=64, seed=0x5EED0190)
    g, o, _ = run(sp, nv=nv)
    assert_scores_close(g, o, "held scores, multi-tile workgroups")
    for r in range(3):
        assert np.all(np.isneginf(g[r, nv[r]:])), f"row {r}: keys past the visible count"


@pytest.mark.parametrize("spread", [False, True])
@pytest.mark.parametrize("H", [8, 64, 100])
def test_fp8_keys_summation_bound(H, spread):
    """fp8 keys against bf16 queries: the query enters the fp8 MFMA as two E4M3
    halves that add up to it, so the products are exact and only the MFMA's sums
    round.  The GPU score stays within 1e-4 of the absolute condition
    scale_s * sum_h |w_h| sum_i |q_hi k_si| of the fp64 oracle (measured: 3e-6 on the
    workload's distribution, 3e-5 with the spread below), 200 times tighter than the
    general score tolerance; a query rounded to a single E4M3 half is off by 5e-3.
    The halves reproduce every query value of a scale run (the 32 dimensions
    16 j + [0, 16) and 64 + 16 j + [0, 16)) down to 2^-13 of the run's maximum m;
    smaller values may be off by up to 2^-21 m, which the bound adds per element.
    spread: query values scaled by powers of two over 24 binades, so that runs mix
    magnitudes far below their maximum."""
    print("fp8 summation bound", H, spread, flush=True)
    sp = workloads.spec("batched_decode", B=2, S=3001, H=H, seed=0x5EED0150 + H + 7 * spread)
    x = workloads.indexer_inputs(sp)
    if spread:
        rng = np.random.default_rng(0x5EED0151 + H)
        qf = (x["q"].astype(np.uint32) << 16).view(np.float32)
        qf = qf * np.exp2(rng.integers(-20, 5, size=qf.shape)).astype(np.float32)
        x["q"] = (qf.view(np.uint32) >> 16).astype(np.uint16)
    g = li.indexer_score(dev(x["q"], "bf16"), dev(x["w"]), dev(x["k"], "fp8"), dev(x["k_scale"]))
    torch.cuda.synchronize()
    g = g.cpu().numpy().astype(np.float64)
    o = oracle.indexer_score(x["q"], oracle.BF16, x["w"], x["k"], oracle.FP8_E4M3, x["k_scale"])
    lut = np.array([oracle.dec_e4m3(c) for c in range(256)])
    kabs = np.abs(lut[x["k"]])                                   # [B, S, d]
    qabs = np.abs((x["q"].astype(np.uint32) << 16).view(np.float32).astype(np.float64))  # [B, 1, H, d]
    v = np.einsum("bh,bhd->bd", np.abs(x["w"][:, 0].astype(np.float64)), qabs[:, 0])
    cond = x["k_scale"].astype(np.float64) * np.einsum("bsd,bd->bs", kabs, v)
    qr = qabs[:, 0].reshape(qabs.shape[0], H, 2, 4, 16)           # [B, H, half, run, 16]
    m = qr.max(axis=(2, 4), keepdims=True)
    ex = np.floor(np.log2(np.where(m > 0, m, 1.0)))
    e_split = np.where(qr < np.exp2(ex - 13), np.exp2(-21.0) * m, 0.0).reshape(qabs.shape[0], H, 128)
    vs = np.einsum("bh,bhd->bd", np.abs(x["w"][:, 0].astype(np.float64)), e_split)
    split = x["k_scale"].astype(np.float64) * np.einsum("bsd,bd->bs", kabs, vs)
    err = np.abs(g - o)
    bound = 1e-4 * cond + split + 1e-6 * np.abs(o)
    assert (err <= bound).all(), f"H={H}: worst error / condition {np.max(err / np.maximum(cond, 1e-300)):.3e}"


# H = 12: three groups of four heads; H = 7: one group and three single heads;
# S = 1500 and 1001: a ragged last workgroup of 64 keys
@pytest.mark.parametrize("combo,H,S", [(("f32", "f32"), 12, 1500), (("f32", "fp8"), 12, 1500),
                                       (("f32", "bf16"), 12, 1500), (("bf16", "f32"), 12, 1500),
                                       (("f32", "f32"), 7, 1001), (("bf16", "f32"), 7, 1001)])
def test_fp32_paths(combo, H, S):
    qt, kt = combo
    print("fp32 path", combo, H, S, flush=True)
    sp = workloads.spec("tiny_decode", B=2, S=S, H=H, q=qt, key=kt, seed=0x5EED0200 + H)
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


@pytest.mark.parametrize("B,T,S,H", [(2, 17, 1000, 64), (1, 40, 3001, 100), (3, 64, 513, 8), (1, 16, 5000, 32)])
def test_prefill_fp8_keys(B, T, S, H):
    # fp8 keys at prefill shapes: the tiled kernel widens the codes to bf16 on their
    # way into LDS and multiplies each key's head sum by its scale; ragged rows, key
    # tails and visible counts in [0, S]
    print("prefill fp8 keys", B, T, S, H, flush=True)
    sp = workloads.spec("prefill_chunk", B=B, T=T, S=S, H=H, key="fp8", seed=0x5EED0D00 + T + S)
    rng = np.random.default_rng(T * S + 1)
    nv = rng.integers(0, S + 1, B * T).astype(np.int32)
    nv[0], nv[-1] = 0, S
    g, o, _ = run(sp, nv=nv)
    assert_scores_close(g, o, f"prefill fp8 B={B} T={T} S={S} H={H}")
    for r in range(B * T):
        assert np.isneginf(g[r, nv[r]:]).all() and np.isfinite(g[r, : nv[r]]).all()


def test_prefill_fp8_every_code():
    """Exact widening of every finite E4M3 code in every byte position of a chunk:
    query row r has q = +1 (head 0) and -1 (head 1) at dimension d_r and zeros
    elsewhere, w = (1, 2^-16), scales powers of two, so each score is one decoded
    code, ReLU'd from either side, with no rounding anywhere: the GPU's fp32 scores
    must equal the oracle's (which decodes the codes itself) bit for bit."""
    print("prefill fp8 every code", flush=True)
    T, H = 16, 2
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)  # 0x7F, 0xFF are NaN
    S = 2 * len(codes)
    d_r = np.array([8 * r + (r % 8) for r in range(T)])  # every byte offset of a chunk, several chunks
    k = codes[(np.arange(S)[:, None] + 7 * np.arange(128)[None, :]) % len(codes)][None]  # [1, S, 128]
    ks = np.ldexp(1.0, (np.arange(S) % 5) - 2).astype(np.float32)[None]
    qf = np.zeros((1, T, H, 128), np.float32)
    for r in range(T):
        qf[0, r, 0, d_r[r]] = 1.0
        qf[0, r, 1, d_r[r]] = -1.0
    q = (qf.view(np.uint32) >> 16).astype(np.uint16)  # exact bf16 of +-1 and 0
    w = np.tile(np.array([1.0, 2.0 ** -16], np.float32), (1, T, 1))
    g = li.indexer_score(dev(q, "bf16"), dev(w), dev(k, "fp8"), dev(ks))
    torch.cuda.synchronize()
    o = oracle.indexer_score(q, oracle.BF16, w, k, oracle.FP8_E4M3, ks)
    assert np.array_equal(g.cpu().numpy(), o.astype(np.float32))
    # every code reached some row at each of its byte offsets
    seen = {(int(k[0, s, d_r[r]]), int(d_r[r] % 8)) for r in range(T) for s in range(S)}
    assert len(seen) == len(codes) * 8


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
