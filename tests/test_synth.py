"""Checks of the seeded input generators: storage-format rounding, determinism,
random access and distribution moments."""
import math

import numpy as np
import torch

import synth
from synth import workloads


def test_bf16_round_to_nearest_even():
    rng = np.random.default_rng(0)
    xs = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000),
                         [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0, -0.0]])
    for x in xs:
        b = synth.bf16_rne(x)
        v = float(np.uint32(b << 16).view(np.float32))
        # neighbours one bf16 step away on either side are no closer
        for nb in ((b + 1) & 0xFFFF, (b - 1) & 0xFFFF):
            u = float(np.uint32(nb << 16).view(np.float32))
            if math.isfinite(u) and (u > 0) == (v > 0):
                assert abs(u - x) >= abs(v - x)
                if abs(u - x) == abs(v - x):
                    assert (b & 1) == 0
    assert synth.bf16_rne(1.0 + 2 ** -8) == 0x3F80  # tie -> even
    assert synth.bf16_rne(1.0 + 3 * 2 ** -8) == 0x3F82


def test_e4m3_round_to_nearest_even():
    vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    finite = [(c, v) for c, v in enumerate(vals) if np.isfinite(v)]
    for c, v in finite:
        if c != 0x80:
            assert synth.e4m3_rne(v) == c
    assert synth.e4m3_rne(1000.0) == 0x7E and synth.e4m3_rne(-449.0) == 0xFE
    pos = sorted(v for c, v in finite if v >= 0)
    rng = np.random.default_rng(1)
    for x in rng.uniform(0, 448, 3000):
        c = synth.e4m3_rne(x)
        got = vals[c]
        best = min(abs(p - x) for p in pos)
        assert abs(got - x) == best


def test_random_access_and_determinism():
    a = synth.normal_bf16(7, 3, (1000,))
    b = synth.normal_bf16(7, 3, (501,), off=499)
    assert np.array_equal(a[499:], b)
    rows = synth.normal_bf16_rows(7, 3, np.array([3, 0, 7]), 100)
    full = synth.normal_bf16(7, 3, (10, 100))
    assert np.array_equal(rows, full[[3, 0, 7]])
    c1, s1 = synth.fp8_rows(5, 2, 40, 128)
    c2, s2 = synth.fp8_rows(5, 2, 10, 128, row_off=30)
    assert np.array_equal(c1[30:], c2) and np.array_equal(s1[30:], s2)
    assert not np.array_equal(synth.normal_f32(7, 3, (64,)), synth.normal_f32(7, 4, (64,)))


def test_moments():
    x = synth.normal_f64(11, 1, (400000,))
    assert abs(x.mean()) < 0.01 and abs(x.var() - 1) < 0.01
    assert abs((x ** 4).mean() - 3) < 0.05
    u = synth.uniform_f32(11, 2, (400000,), 0.0, 1.0)
    assert 0 <= u.min() and u.max() < 1 and abs(u.mean() - 0.5) < 0.005


def test_fp8_rows_scale_rule():
    codes, scales = synth.fp8_rows(3, 3, 50, 128)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    # each row's largest |code| is 448 (the row max maps to the format max)
    assert np.all(np.abs(vals).max(axis=1) == 448.0)
    x = synth.normal_f64(3, 3, (50, 128))
    np.testing.assert_allclose(vals * scales[:, None], x, rtol=2 ** -3, atol=scales.max() * 2 ** -9)


def test_causal_visibility():
    nv = workloads.causal_nv(131072, 4096)
    assert nv[0] == 130049 and nv[-1] == 131072 and int(nv.astype(np.int64).sum()) == 534775808
