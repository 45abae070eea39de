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


# ---- derivative of the recurrence (reverse time) ------------------------------------------------
def _loss(xs, fs, h0, dh, gl):
    """L = sum_t dh_t h_t + gl h_{T-1}, with h from the exact closed form above."""
    h = _closed_form(xs, fs, h0)
    return sum(Fraction(a) * b for a, b in zip(dh, h)) + Fraction(gl) * h[-1]


def test_scan_bwd_is_the_exact_derivative():
    """L is affine in every single x_s, f_s and h_0 (the closed form is multilinear), so
    L(v + 1) - L(v) is the exact partial derivative. With dyadic inputs of a few bits the
    oracle's binary64 arithmetic is exact and must equal it."""
    g = synth.rng(31)
    for T in range(1, 7):
        xs = (g.integers(-16, 17, size=T) / 16.0).tolist()
        fs = (g.integers(0, 9, size=T) / 8.0).tolist()
        dh = (g.integers(-8, 9, size=T) / 8.0).tolist()
        h0 = g.integers(-4, 5) / 4.0
        gl = g.integers(-4, 5) / 4.0
        h = oracle.hgrn_scan(np.array(xs).reshape(1, T, 1), np.array(fs).reshape(1, T, 1), np.array([[h0]]))
        dx, df, dh0 = oracle.hgrn_scan_bwd(np.array(fs).reshape(1, T, 1), h, np.array(dh).reshape(1, T, 1),
                                           np.array([[h0]]), np.array([[gl]]))
        base = _loss(xs, fs, h0, dh, gl)
        for s in range(T):
            up = list(xs)
            up[s] += 1
            assert Fraction(dx[0, s, 0]) == _loss(up, fs, h0, dh, gl) - base, (T, s, "x")
            up = list(fs)
            up[s] += 1
            assert Fraction(df[0, s, 0]) == _loss(xs, up, h0, dh, gl) - base, (T, s, "f")
        assert Fraction(dh0[0, 0]) == _loss(xs, fs, h0 + 1, dh, gl) - base, (T, "h0")


def test_scan_bwd_adjoint_identity():
    """For fixed f the map (x, h0) -> h is linear, so <dh, h> + <dh_last, h_last> = <dx, x> + <dh0, h0>."""
    g = synth.rng(32)
    x = g.standard_normal((3, 40, 5))
    f = g.uniform(0, 1, (3, 40, 5))
    h0 = g.standard_normal((3, 5))
    dh = g.standard_normal((3, 40, 5))
    gl = g.standard_normal((3, 5))
    h = oracle.hgrn_scan(x, f, h0)
    dx, df, dh0 = oracle.hgrn_scan_bwd(f, h, dh, h0, gl)
    lhs = np.sum(dh * h) + np.sum(gl * h[:, -1])
    rhs = np.sum(dx * x) + np.sum(dh0 * h0)
    assert abs(lhs - rhs) <= 1e-12 * (np.sum(np.abs(dh * h)) + np.sum(np.abs(gl * h[:, -1])))


def test_scan_bwd_limits():
    """f = 0: no step reaches back, dx = dh (dh_last joins the last step), dh0 = 0. f = 1: dx is
    the reverse cumulative sum of dh plus dh_last, and dh0 = dx_0."""
    g = synth.rng(33)
    x = g.integers(-64, 64, size=(2, 7, 3)) / 8.0
    h0 = g.integers(-8, 8, size=(2, 3)) / 4.0
    dh = g.integers(-64, 64, size=(2, 7, 3)) / 8.0
    gl = g.integers(-8, 8, size=(2, 3)) / 4.0
    zero = np.zeros_like(x)
    h = oracle.hgrn_scan(x, zero, h0)
    dx, df, dh0 = oracle.hgrn_scan_bwd(zero, h, dh, h0, gl)
    want = dh.copy()
    want[:, -1] += gl
    assert np.array_equal(dx, want)
    h_prev = np.concatenate([h0[:, None, :], h[:, :-1]], axis=1)
    assert np.array_equal(df, want * h_prev)
    assert np.array_equal(dh0, np.zeros_like(h0))
    one = np.ones_like(x)
    h = oracle.hgrn_scan(x, one, h0)
    dx, df, dh0 = oracle.hgrn_scan_bwd(one, h, dh, h0, gl)
    want = np.flip(np.cumsum(np.flip(dh, axis=1), axis=1), axis=1) + gl[:, None, :]
    assert np.array_equal(dx, want)
    assert np.array_equal(dh0, want[:, 0])


def test_scan_bwd_empty_sequence_passes_dh_last():
    gl = np.arange(6.0).reshape(2, 3)
    e = np.zeros((2, 0, 3))
    dx, df, dh0 = oracle.hgrn_scan_bwd(e, e, e, np.ones((2, 3)), gl)
    assert dx.shape == (2, 0, 3) and np.array_equal(dh0, gl)
