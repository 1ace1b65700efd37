"""GPU parity of the paged caches (li_indexer_score_paged, li_indexer_topk_paged,
li_sparse_attn_gather_paged): the same logical keys and rows, scattered over pool
pages in a random order among garbage pages, give bit for bit the results of the
unpaged calls, and those match the oracle's paged reads within the usual rules."""
import numpy as np
import pytest
import torch

import lightning_indexer_top_amd as li
import oracle
import synth
from synth import workloads
from helpers import assert_attn_close, assert_scores_close, assert_topk_band, bf16_host, dev

pytestmark = pytest.mark.gpu

PAGE = 64


def paged_keys(codes, scales, extra, seed):
    """codes [B, S, 128] uint8, scales [B, S] -> device pools and page table."""
    B, S = scales.shape
    P = (S + PAGE - 1) // PAGE
    rng = np.random.default_rng(seed)
    num = B * P + extra
    perm = rng.permutation(num)[:B * P].reshape(B, P)
    kpool = rng.integers(0, 0x7E, (num, PAGE, 128)).astype(np.uint8)
    spool = rng.uniform(0.5, 2.0, (num, PAGE)).astype(np.float32)
    for b in range(B):
        for p in range(P):
            n = min(PAGE, S - p * PAGE)
            kpool[perm[b, p], :n] = codes[b, p * PAGE:p * PAGE + n]
            spool[perm[b, p], :n] = scales[b, p * PAGE:p * PAGE + n]
    table = np.concatenate([perm, np.full((B, 2), num - 1)], axis=1).astype(np.int32)
    return kpool, spool, table


@pytest.mark.parametrize("B,S,H,k", [(3, 20037, 64, 512), (2, 40000, 32, 512), (4, 5000, 128, 64),
                                     (8, 131072, 64, 512), (2, 100, 64, 16), (3, 30001, 8, 256)])
def test_paged_indexer_equals_unpaged(B, S, H, k):
    print("paged indexer", B, S, H, k, flush=True)
    sp = workloads.spec("batched_decode", B=B, S=S, H=H, seed=0x5EED0D00 + S + H)
    x = workloads.indexer_inputs(sp)
    kpool, spool, table = paged_keys(x["k"], x["k_scale"], 9, S)
    q, w = dev(x["q"], "bf16"), dev(x["w"])
    kp, sp_, tb = dev(kpool, "fp8"), dev(spool), dev(table)
    for nv in (None, np.array(([S, 0, 1, S - 63, 511, 513, 64, S // 2] * B)[:B], np.int32)):
        nvd = dev(nv) if nv is not None else None
        g = li.indexer_score_paged(q, w, kp, sp_, tb, S, nvd)
        u = li.indexer_score(q, w, dev(x["k"], "fp8"), dev(x["k_scale"]), nvd)
        gi, gv = li.indexer_topk_paged(q, w, kp, sp_, tb, S, k, nvd)
        ui, uv = li.indexer_topk(q, w, dev(x["k"], "fp8"), k, dev(x["k_scale"]), nvd)
        torch.cuda.synchronize()
        assert torch.equal(g, u), "paged scores differ from unpaged"
        assert torch.equal(gi, ui) and torch.equal(gv, uv), "paged selection differs from unpaged"
        if S <= 40000:
            o = oracle.indexer_score_paged(x["q"], oracle.BF16, x["w"], kpool, spool, table, S, nv)
            assert_scores_close(g.cpu().numpy(), o, "paged scores")
            assert_topk_band(gi.cpu().numpy(), o, k, nv, "paged top-k")


@pytest.mark.parametrize("B,Hq,S,k", [(2, 128, 3000, 512), (3, 64, 900, 100), (1, 32, 70, 70),
                                      (2, 96, 5000, 2048)])
def test_paged_attention_equals_unpaged(B, Hq, S, k):
    print("paged attention", B, Hq, S, k, flush=True)
    kv = synth.normal_bf16(0x5EED0D10 + S, 5, (B, S, 576))
    qa = synth.normal_bf16(0x5EED0D10 + S, 6, (B, Hq, 576))
    rng = np.random.default_rng(S)
    num = B * S + 33
    slots = rng.permutation(num)[:B * S].reshape(B, S)
    pool = rng.integers(0, 0x3F80, (num, 576)).astype(np.uint16)
    for b in range(B):
        pool[slots[b]] = kv[b]
    table = np.concatenate([slots, np.zeros((B, 5), np.int64)], axis=1).astype(np.int32)
    idx = np.sort(np.stack([rng.choice(S, k, replace=False) for _ in range(B)]), axis=1).astype(np.int32)
    idx[0, 1] = -1
    if k > 3:
        idx[-1, 2] = S + 10  # outside [0, S): selects nothing
    tau = 1 / np.sqrt(192)
    g, gl = li.sparse_attn_gather_paged(dev(qa, "bf16"), dev(pool, "bf16"), dev(table), S, dev(idx), tau)
    u, ul = li.sparse_attn_gather(dev(qa, "bf16"), dev(kv, "bf16"), dev(idx), tau)
    torch.cuda.synchronize()
    assert torch.equal(g, u) and torch.equal(gl, ul), "paged attention differs from unpaged"
    o, ol = oracle.sparse_attn_paged(qa, pool, table, idx, 512, tau)
    assert_attn_close(bf16_host(g), o, "paged attention")
    np.testing.assert_allclose(gl.cpu().numpy(), ol, rtol=1e-3, atol=1e-3)
