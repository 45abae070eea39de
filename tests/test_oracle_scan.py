"""Pins for the oracle's HGRN recurrence: exact rationals, closed forms, limits.

With dyadic inputs of a few bits every product and sum is exact in binary64,
so the oracle must equal the unrolled closed form
    h_T = sum_s (prod_{r=s+1..T} f_r) x_s + (prod_r f_r) h_0
evaluated in exact rationals (Python fractions).
"""
from fractions import Fraction

import numpy as np

import oracle
from ternary_weight_matmul_amd import synth


def _closed_form(xs, fs, h0):
    out = []
    for T in range(len(xs)):
        acc = Fraction(h0)
        for r in range(T + 1):
            acc *= Fraction(fs[r])
        for s in range(T + 1):
            p = Fraction(xs[s])
            for r in range(s + 1, T + 1):
                p *= Fraction(fs[r])
            acc += p
        out.append(acc)
    return out


def test_scan_matches_exact_unrolled_sum():
    g = synth.rng(21)
    for T in range(1, 9):
        xs = g.integers(-16, 17, size=T) / 16.0
        fs = g.integers(0, 9, size=T) / 8.0
        h0 = g.integers(-4, 5) / 4.0
        h = oracle.hgrn_scan(xs.reshape(1, T, 1), fs.reshape(1, T, 1), np.array([[h0]]))
        exact = _closed_form(xs.tolist(), fs.tolist(), h0)
        assert [Fraction(v) for v in h[0, :, 0].tolist()] == exact


def test_constant_gate_geometric_series():
    h = oracle.hgrn_scan(np.ones((1, 5, 1)), np.full((1, 5, 1), 0.5))
    assert h[0, :, 0].tolist() == [1.0, 1.5, 1.75, 1.875, 1.9375]


def test_zero_gate_is_identity_and_unit_gate_is_cumsum():
    g = synth.rng(22)
    x = g.integers(-64, 64, size=(2, 7, 3)) / 8.0
    h0 = g.integers(-8, 8, size=(2, 3)) / 4.0
    assert np.array_equal(oracle.hgrn_scan(x, np.zeros_like(x), h0), x)
    assert np.array_equal(oracle.hgrn_scan(x, np.ones_like(x), h0), h0[:, None, :] + np.cumsum(x, axis=1))


def test_channels_and_batches_are_independent():
    g = synth.rng(23)
    x = g.standard_normal((3, 11, 4))
    f = g.uniform(0, 1, (3, 11, 4))
    h = oracle.hgrn_scan(x, f)
    for b in range(3):
        for c in range(4):
            hc = oracle.hgrn_scan(x[b:b + 1, :, c:c + 1], f[b:b + 1, :, c:c + 1])
            assert np.array_equal(hc[0, :, 0], h[b, :, c])


def test_split_sequence_carries_state():
    g = synth.rng(24)
    x = g.standard_normal((2, 20, 5))
    f = g.uniform(0, 1, (2, 20, 5))
    h = oracle.hgrn_scan(x, f)
    h1 = oracle.hgrn_scan(x[:, :9], f[:, :9])
    h2 = oracle.hgrn_scan(x[:, 9:], f[:, 9:], h1[:, -1])
    assert np.array_equal(np.concatenate([h1, h2], axis=1), h)
