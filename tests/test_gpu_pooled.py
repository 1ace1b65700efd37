"""GPU parity of the pooled-key indexer (li_pool_keys, li_pooled_indexer_topk)
against the oracle: pooled fp8 codes and scales bit for bit (the pooling decides
integer codes, taken in the same fp32 steps on both sides), the selected blocks
within the near-tie band of the oracle's block scores and equal to the oracle's
selection of the GPU's own block scores, and the tokens the exact expansion of
those blocks."""
import numpy as np
import pytest
import torch

import lightning_indexer_top_amd as li
import oracle
import synth
from synth import workloads
from helpers import assert_topk_band, dev

pytestmark = pytest.mark.gpu


def gpu_pool(k_tok, pool):
    codes, scales = li.pool_keys(dev(k_tok, "bf16"), pool)
    torch.cuda.synchronize()
    return codes.view(torch.uint8).cpu().numpy(), scales.cpu().numpy()


@pytest.mark.parametrize("pool", [1, 2, 4, 8])
def test_pool_keys_bit_exact(pool):
    print("pool keys", pool, flush=True)
    B, L = 3, 8 * 501 + 5  # an incomplete last block
    k = synth.normal_bf16(0x5EED0A00 + pool, 3, (B, L, 128))
    # crafted blocks: a zero block, one large value among tiny ones (subnormal
    # codes), opposite pairs that cancel to zero
    k[0, :8] = 0
    tiny = synth.normal_bf16(0x5EED0A10, 3, (8, 128), 1e-4)
    k[1, 8:16] = tiny
    k[1, 8:16, 5] = synth.bf16_rne(3.0)
    k[2, 16:24] = k[2, 24:32]
    k[2, 17:24:2] = k[2, 16:24:2] ^ 0x8000
    codes, scales = gpu_pool(k, pool)
    o_codes, o_scales = oracle.pool_keys(k, pool)
    assert codes.shape == o_codes.shape
    assert np.array_equal(scales, o_scales), "scales differ"
    bad = codes != o_codes
    assert not bad.any(), f"{bad.sum()} codes differ (first at {np.argwhere(bad)[0].tolist()})"


def test_pool_keys_short_sequences():
    print("pool keys short", flush=True)
    k = synth.normal_bf16(0x5EED0A20, 3, (2, 3, 128))
    codes, scales = li.pool_keys(dev(k, "bf16"), 4)  # no complete block: nothing written
    assert codes.shape == (2, 0, 128) and scales.shape == (2, 0)


def pooled_case(sp, nv_tokens=None):
    x = workloads.pooled_inputs(sp)
    pool, k = sp["pool"], sp["topk"]
    q, w = dev(x["q"], "bf16"), dev(x["w"])
    codes, scales = li.pool_keys(dev(x["k_tokens"], "bf16"), pool)
    nvd = dev(nv_tokens) if nv_tokens is not None else None
    idx, val = li.pooled_indexer_topk(q, w, codes, scales, pool, k, nvd)
    # the GPU's own block scores (li_indexer_score on the pooled keys)
    B, T = sp["B"], sp["T"]
    Sp = codes.shape[1]
    nvb = None
    if nv_tokens is not None:
        nvb = np.minimum(np.maximum(nv_tokens, 0) // pool, Sp).astype(np.int32)
    gs = li.indexer_score(q, w, codes, scales, dev(nvb) if nvb is not None else None)
    torch.cuda.synchronize()
    return x, codes.view(torch.uint8).cpu().numpy(), scales.cpu().numpy(), idx.cpu().numpy(), \
        val.cpu().numpy(), gs.cpu().numpy().astype(np.float64), nvb


def check_pooled(sp, nv_tokens=None):
    pool, k = sp["pool"], sp["topk"]
    x, codes, scales, idx, val, gs, nvb = pooled_case(sp, nv_tokens)
    o_codes, o_scales = oracle.pool_keys(x["k_tokens"], pool)
    assert np.array_equal(codes, o_codes) and np.array_equal(scales, o_scales)
    R = sp["B"] * sp["T"]
    # blocks: every pool-th token, the rest its expansion
    blocks = idx[:, ::pool]
    exp = np.where(blocks[:, :, None] >= 0, blocks[:, :, None] + np.arange(pool), -1).reshape(R, -1)
    assert np.array_equal(idx, exp), "tokens are not the expansion of the blocks"
    assert np.all((blocks == -1) | (blocks % pool == 0))
    blk = np.where(blocks >= 0, blocks // pool, -1)
    # same precision decision: the oracle's selection of the GPU's block scores
    r_idx, r_val = oracle.topk(gs, k, nvb)
    assert np.array_equal(blk, r_idx)
    fin = r_idx >= 0
    assert np.array_equal(val.astype(np.float64)[fin], r_val[fin])
    # against the oracle's own pooled selection: band rule on the block scores
    o = oracle.indexer_score(x["q"], oracle.BF16, x["w"], o_codes, oracle.FP8_E4M3, o_scales, nvb)
    assert_topk_band(blk, o, k, nvb, "pooled blocks")


@pytest.mark.parametrize("B,L,pool,k", [(3, 4 * 5000 + 3, 4, 512), (2, 2 * 9000, 2, 64), (4, 8 * 3000, 8, 100),
                                        (2, 4 * 70000, 4, 512), (3, 1000, 1, 2048)])
def test_pooled_selection(B, L, pool, k):
    print("pooled select", B, L, pool, k, flush=True)
    sp = workloads.spec("pooled_decode", B=B, L=L, pool=pool, topk=k, seed=0x5EED0B00 + L + pool)
    check_pooled(sp)


def test_pooled_visible_tokens():
    print("pooled nv", flush=True)
    sp = workloads.spec("pooled_decode", B=6, L=4 * 20000, pool=4, topk=512, seed=0x5EED0B77)
    nv = np.array([4 * 20000, 0, 3, 4 * 300 + 3, 4 * 512, 4 * 10000 + 1], np.int32)
    check_pooled(sp, nv)


def test_pooled_decode_full_size():
    sp = workloads.spec("pooled_decode")
    B, L, pool, k = sp["B"], sp["L"], sp["pool"], sp["topk"]
    print("full size pooled_decode", B, L, flush=True)
    x, codes, scales, idx, val, gs, _ = pooled_case(sp)
    for b in (0, B - 1):
        print("oracle pooling, sequence", b, flush=True)
        oc, os_ = oracle.pool_keys(x["k_tokens"][b:b + 1], pool)
        assert np.array_equal(codes[b:b + 1], oc) and np.array_equal(scales[b:b + 1], os_)
    blocks = idx[:, ::pool]
    assert (blocks >= 0).all() and np.all(np.diff(blocks, axis=1) > 0)
    blk = blocks // pool
    r_idx, _ = oracle.topk(gs, k)
    assert np.array_equal(blk, r_idx)
    print("oracle block scores, all rows", flush=True)
    o = oracle.indexer_score(x["q"], oracle.BF16, x["w"], codes, oracle.FP8_E4M3, scales)
    assert_topk_band(blk, o, k, None, "pooled_decode blocks")
