"""GPU parity of li_sparse_attn_gather against the fp64 oracle (per (b, head) max
error / max |out| <= 1e-2; lse to 1e-3 relative), including skipped entries,
a ragged last chunk and repeated rows."""
import math

import numpy as np
import pytest
import torch

import lightning_indexer_top_amd as li
import oracle
import synth
from helpers import assert_attn_close, bf16_host, dev

pytestmark = pytest.mark.gpu


def run(B, Hq, S, k, seed, idx=None, tau=1 / math.sqrt(192)):
    q = synth.normal_bf16(seed, 6, (B, Hq, 576))
    kv = synth.normal_bf16(seed, 5, (B, S, 576))
    if idx is None:
        rng = np.random.default_rng(seed)
        idx = np.stack([rng.choice(S, k, replace=False) for _ in range(B)]).astype(np.int32)
    out, lse = li.sparse_attn_gather(dev(q, "bf16"), dev(kv, "bf16"), dev(idx), tau)
    torch.cuda.synchronize()
    o_out, o_lse = oracle.sparse_attn(q, kv, np.where((idx >= 0) & (idx < S), idx, -1), 512, tau)
    return bf16_host(out), lse.cpu().numpy(), o_out, o_lse


# k = 1 and 33: the second half of a workgroup takes no chunk or a one-row chunk;
# k = 64: one full chunk each; k = 2048: 32 chunks a half
@pytest.mark.parametrize("B,Hq,S,k", [(2, 128, 3000, 512), (3, 32, 500, 100), (1, 64, 5000, 2048), (2, 96, 64, 1),
                                      (2, 32, 700, 33), (1, 128, 2000, 64), (2, 64, 700, 33), (2, 128, 64, 1),
                                      (3, 128, 900, 300)])
def test_matches_oracle(B, Hq, S, k):
    print("attn", B, Hq, S, k, flush=True)
    g, gl, o, ol = run(B, Hq, S, k, seed=0x5EED0800 + k)
    assert_attn_close(g, o)
    np.testing.assert_allclose(gl, ol, rtol=1e-3, atol=1e-3)


def test_skipped_and_repeated_entries():
    print("attn skip", flush=True)
    S = 300
    rng = np.random.default_rng(3)
    idx = rng.integers(0, S, (2, 200)).astype(np.int32)  # repeats allowed
    idx[0, ::7] = -1
    idx[1, 150:] = -1
    idx[1, 10] = S + 5                                   # out of range counts as skipped
    g, gl, o, ol = run(2, 64, S, 200, seed=0x5EED0900, idx=idx)
    assert_attn_close(g, o)
    np.testing.assert_allclose(gl, ol, rtol=1e-3, atol=1e-3)


@pytest.mark.parametrize("Hq", [32, 128])
def test_nothing_selected(Hq):
    print("attn empty", Hq, flush=True)
    idx = -np.ones((1, 40), np.int32)
    g, gl, o, ol = run(1, Hq, 100, 40, seed=0x5EED0A00, idx=idx)
    assert (g == 0).all() and np.isneginf(gl).all()


def bf16_bits(x):
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("pos,scale", [(10, 4.0), (40, 4.0), (200, 2.0), (300, 0.6), (509, 4.0)])
def test_late_dominant_row(pos, scale):
    """A selected row planted as a multiple of one query makes that head's logit jump
    far above everything seen in the earlier chunks (and others' by less), so the
    running softmax reference has to move mid-sequence; sequence 1 also starts with
    two chunks of skipped entries.  Chunks (32 selected rows) alternate between the two
    halves of the workgroup, so positions 10 and 200 move a reference in the first half,
    40, 300 and 509 in the second, and the final merge rescales the other half."""
    print("attn dominant", pos, scale, flush=True)
    B, Hq, S, k, seed = 2, 64, 4000, 512, 0x5EED0B00 + pos
    tau = 1 / math.sqrt(192)
    q = synth.normal_bf16(seed, 6, (B, Hq, 576))
    kv = synth.normal_bf16(seed, 5, (B, S, 576))
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(S, k, replace=False) for _ in range(B)]).astype(np.int32)
    idx[1, :64] = -1
    for b, h in ((0, 5), (1, 37)):
        row = idx[b, pos]
        planted = (np.asarray(q[b, h], np.uint32) << 16).view(np.float32)
        kv[b, row] = bf16_bits(planted * scale)
    out, lse = li.sparse_attn_gather(dev(q, "bf16"), dev(kv, "bf16"), dev(idx), tau)
    torch.cuda.synchronize()
    o_out, o_lse = oracle.sparse_attn(q, kv, np.where((idx >= 0) & (idx < S), idx, -1), 512, tau)
    assert_attn_close(bf16_host(out), o_out)
    np.testing.assert_allclose(lse.cpu().numpy(), o_lse, rtol=1e-3, atol=1e-3)
