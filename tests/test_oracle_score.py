"""Pins of the oracle's indexer score (O1) against hand-worked values, exact
rationals, closed forms and invariants -- none of them re-runs the oracle's own
formula.  The score follows the "Long context" lecture, section "The
Architectural Answer", paragraph "Stage 1, the lightning indexer"."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _f32(a):
    return np.asarray(a, np.float32)


def test_hand_worked_scores():
    cases = json.load(open(os.path.join(GOLD, "score_hand.json")))["cases"]
    for c in cases:
        q, w, k = _f32(c["q"]), _f32(c["w"]), _f32(c["k"])
        got = oracle.indexer_score(q, oracle.F32, w, k, oracle.F32)
        assert np.array_equal(got, np.asarray(c["scores"], np.float64)), c["note"]


def test_decoders_match_torch_formats():
    # bf16 and OCP fp8 E4M3FN decoding agrees with torch's own dtypes for every code
    codes8 = np.arange(256, dtype=np.uint8)
    ref8 = torch.from_numpy(codes8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got8 = np.array([oracle.dec_e4m3(c) for c in codes8])
    finite = ~np.isnan(ref8)
    assert np.array_equal(np.isnan(got8), np.isnan(ref8))
    assert np.array_equal(got8[finite], ref8[finite])
    assert oracle.dec_e4m3(0x7E) == 448.0 and oracle.dec_e4m3(0x01) == 2.0 ** -9 and oracle.dec_e4m3(0x08) == 2.0 ** -6
    rng = np.random.default_rng(1)
    codes16 = np.concatenate([rng.integers(0, 65536, 4000), [0, 0x8000, 0x3F80, 0x7F7F, 0x0001]]).astype(np.uint16)
    ref16 = torch.from_numpy(codes16.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got16 = np.array([oracle.dec_bf16(c) for c in codes16])
    ok = ~np.isnan(ref16)
    assert np.array_equal(got16[ok], ref16[ok])


def _exact(v, kind):
    """Exact rational value of a stored element (decoded through numpy/torch)."""
    if kind == "f32":
        return Fraction(float(np.float32(v)))
    if kind == "bf16":
        return Fraction(float(np.uint32(int(v) << 16).view(np.float32)))
    raise ValueError(kind)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_exact_rational_brute_force(seed):
    rng = np.random.default_rng(seed)
    B, T, S, H, d = 1, 2, 17, 3, 8
    # fp8 keys with scales, bf16 queries: compare with the exact rational score
    kc = rng.integers(0, 256, (B, S, d)).astype(np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x30  # no NaN codes
    ks = (rng.random((B, S)) + 0.5).astype(np.float32)
    q = np.array([synth.bf16_rne(x) for x in rng.standard_normal(B * T * H * d)], np.uint16).reshape(B, T, H, d)
    w = rng.random((B, T, H)).astype(np.float32)
    got = oracle.indexer_score(q, oracle.BF16, w, kc, oracle.FP8_E4M3, ks)
    kv = torch.from_numpy(kc).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for t in range(T):
        for s in range(S):
            acc = Fraction(0)
            mag = Fraction(0)
            for h in range(H):
                dot = sum(_exact(q[0, t, h, j], "bf16") * Fraction(kv[0, s, j]) * Fraction(float(ks[0, s]))
                          for j in range(d))
                absdot = sum(abs(_exact(q[0, t, h, j], "bf16") * Fraction(kv[0, s, j]) * Fraction(float(ks[0, s])))
                             for j in range(d))
                acc += Fraction(float(w[0, t, h])) * max(dot, Fraction(0))
                mag += Fraction(float(w[0, t, h])) * absdot
            err = abs(Fraction(got[t, s]) - acc)
            assert err <= mag * Fraction(2 * (d + H), 2 ** 53) + Fraction(1, 2 ** 1000)


def test_integer_inputs_are_exact():
    rng = np.random.default_rng(5)
    B, T, S, H, d = 2, 3, 11, 4, 16
    q = rng.integers(-8, 9, (B, T, H, d)).astype(np.float32)
    w = rng.integers(0, 5, (B, T, H)).astype(np.float32)
    k = rng.integers(-8, 9, (B, S, d)).astype(np.float32)
    got = oracle.indexer_score(q, oracle.F32, w, k, oracle.F32)
    qi, wi, ki = q.astype(np.int64), w.astype(np.int64), k.astype(np.int64)
    dots = np.einsum("bthj,bsj->bths", qi, ki)
    ref = (wi[..., None] * np.maximum(dots, 0)).sum(axis=2).reshape(B * T, S)
    assert np.array_equal(got, ref.astype(np.float64))


def test_closed_forms():
    rng = np.random.default_rng(7)
    B, T, S, H, d = 1, 1, 64, 1, 128
    # H = 1, w = 1, all dots positive -> a plain matrix product
    k = np.abs(rng.standard_normal((B, S, d))).astype(np.float32)
    q = np.abs(rng.standard_normal((B, T, H, d))).astype(np.float32)
    w = np.ones((B, T, H), np.float32)
    got = oracle.indexer_score(q, oracle.F32, w, k, oracle.F32)[0]
    ref = k[0].astype(np.float64) @ q[0, 0, 0].astype(np.float64)
    np.testing.assert_allclose(got, ref, rtol=1e-13)
    # all w = 1 and all dots positive -> (sum_h q_h) . k
    H = 6
    q = np.abs(rng.standard_normal((B, T, H, d))).astype(np.float32)
    w = np.ones((B, T, H), np.float32)
    got = oracle.indexer_score(q, oracle.F32, w, k, oracle.F32)[0]
    ref = k[0].astype(np.float64) @ q[0, 0].astype(np.float64).sum(axis=0)
    np.testing.assert_allclose(got, ref, rtol=1e-13)


def _rand_problem(rng, B=2, T=3, S=40, H=5, d=32):
    q = rng.standard_normal((B, T, H, d)).astype(np.float32)
    w = rng.random((B, T, H)).astype(np.float32)
    k = rng.standard_normal((B, S, d)).astype(np.float32)
    return q, w, k


def test_invariants():
    rng = np.random.default_rng(11)
    q, w, k = _rand_problem(rng)
    base = oracle.indexer_score(q, oracle.F32, w, k, oracle.F32)
    # positive homogeneity (powers of two are exact)
    assert np.array_equal(oracle.indexer_score(q * 4, oracle.F32, w, k, oracle.F32), base * 4)
    assert np.array_equal(oracle.indexer_score(q, oracle.F32, w * 0.5, k, oracle.F32), base * 0.5)
    # key permutation equivariance
    perm = rng.permutation(k.shape[1])
    got = oracle.indexer_score(q, oracle.F32, w, k[:, perm], oracle.F32)
    assert np.array_equal(got, base[:, perm])
    # head permutation (changes only the order of the head sum)
    hp = rng.permutation(q.shape[2])
    got = oracle.indexer_score(q[:, :, hp], oracle.F32, w[:, :, hp], k, oracle.F32)
    np.testing.assert_allclose(got, base, rtol=1e-12, atol=1e-300)
    # appending keys leaves earlier scores unchanged
    k2 = np.concatenate([k, rng.standard_normal((k.shape[0], 9, k.shape[2])).astype(np.float32)], axis=1)
    got = oracle.indexer_score(q, oracle.F32, w, k2, oracle.F32)
    assert np.array_equal(got[:, : k.shape[1]], base)
    # a negative head weight subtracts that head's ReLU
    w2 = w.copy()
    w2[..., 0] = -w2[..., 0]
    got = oracle.indexer_score(q, oracle.F32, w2, k, oracle.F32)
    dots0 = np.einsum("btj,bsj->bts", q[:, :, 0].astype(np.float64), k.astype(np.float64)).reshape(-1, k.shape[1])
    delta = 2 * w[..., 0].reshape(-1, 1).astype(np.float64) * np.maximum(dots0, 0)
    np.testing.assert_allclose(base - got, delta, rtol=1e-9, atol=1e-9)


def test_fp8_scale_folds_out():
    rng = np.random.default_rng(3)
    B, T, S, H, d = 1, 1, 30, 4, 16
    codes, scales = synth.fp8_rows(99, 3, B * S, d)
    q = rng.standard_normal((B, T, H, d)).astype(np.float32)
    w = rng.random((B, T, H)).astype(np.float32)
    kc = codes.reshape(B, S, d)
    one = oracle.indexer_score(q, oracle.F32, w, kc, oracle.FP8_E4M3, np.ones((B, S), np.float32))
    sc = oracle.indexer_score(q, oracle.F32, w, kc, oracle.FP8_E4M3, np.full((B, S), 8.0, np.float32))
    assert np.array_equal(sc, one * 8.0)


def test_causal_mask_and_decode_equivalence():
    rng = np.random.default_rng(13)
    q, w, k = _rand_problem(rng, B=1, T=6, S=50)
    nv = np.array([1, 7, 25, 49, 50, 50], np.int32)
    pre = oracle.indexer_score(q, oracle.F32, w, k, oracle.F32, nv=nv)
    for t in range(6):
        assert np.all(np.isneginf(pre[t, nv[t]:]))
        assert np.all(np.isfinite(pre[t, : nv[t]]))
        one = oracle.indexer_score(q[:, t : t + 1], oracle.F32, w[:, t : t + 1], k[:, : nv[t]], oracle.F32)
        assert np.array_equal(pre[t, : nv[t]], one[0])
