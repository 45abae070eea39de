"""Pins for the oracle's FusedBitLinear derivative under straight-through quantisers.

The straight-through reading makes the backward pass the exact derivative of a surrogate in
which each quantiser's output is replaced by its input where the gradient flows: for dx and
dgain, L(x, gain) = sum dy * ((RMSNorm(x) * gain) W^T) with the dequantised ternary weights W^
held fixed; for dW, L(W) = sum dy * (u^ W^T) with the dequantised activations u^ held fixed.
Central differences of those surrogates (smooth in x and gain, linear in W) pin the oracle's
formulas; the RMSNorm's scale invariance pins the direction of dx.
"""
import numpy as np

import oracle
from ternary_weight_matmul_amd import synth


def _setup(m, k, n, seed, with_gain):
    g = synth.rng(seed)
    x = g.standard_normal((m, k)).astype(np.float32)
    w = (g.standard_normal((n, k)) * 0.02).astype(np.float32)
    dy = g.standard_normal((m, n))
    gain = (1.0 + 0.1 * g.standard_normal(k)).astype(np.float32) if with_gain else None
    t, mu = oracle.ternarize(w)
    return x, w, t, mu, dy, gain


def _norm(x, gain, eps):
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1) + eps)
    return x * r[:, None] * (1.0 if gain is None else gain)


def test_dx_and_dgain_are_derivatives_of_the_surrogate():
    eps = np.float64(np.float32(1e-8))
    for seed, with_gain in ((41, False), (42, True)):
        x, _, t, mu, dy, gain = _setup(3, 32, 5, seed, with_gain)
        w_hat = t.astype(np.float64) / np.float64(oracle.weight_scale(mu))
        gain64 = None if gain is None else gain.astype(np.float64)
        dx, _, dgain = oracle.bitlinear_bwd(x, t, mu, dy, gain, 1e-8)

        def loss(xv, gv):
            return np.sum(dy * (_norm(xv, gv, eps) @ w_hat.T))

        x64 = x.astype(np.float64)
        h = 1e-6
        num = np.zeros_like(x64)
        for i in range(x64.shape[0]):
            for j in range(x64.shape[1]):
                e = np.zeros_like(x64)
                e[i, j] = h
                num[i, j] = (loss(x64 + e, gain64) - loss(x64 - e, gain64)) / (2 * h)
        assert np.allclose(dx, num, rtol=1e-6, atol=1e-8 * np.abs(num).max()), seed
        g0 = np.ones(x.shape[1]) if gain64 is None else gain64
        numg = np.zeros_like(g0)
        for j in range(g0.size):
            e = np.zeros_like(g0)
            e[j] = h
            numg[j] = (loss(x64, g0 + e) - loss(x64, g0 - e)) / (2 * h)
        assert np.allclose(dgain, numg, rtol=1e-6, atol=1e-8 * np.abs(numg).max()), seed


def test_dw_is_the_derivative_of_the_linear_surrogate():
    x, w, t, mu, dy, _ = _setup(4, 48, 6, 43, False)
    q, s, _ = oracle.quantize(x)
    u_hat = q.astype(np.float64) / s.astype(np.float64)[:, None]
    _, dw, _ = oracle.bitlinear_bwd(x, t, mu, dy)
    w64 = w.astype(np.float64)

    def loss(wv):
        return np.sum(dy * (u_hat @ wv.T))

    num = np.zeros_like(w64)
    for i in range(w64.shape[0]):
        for j in range(w64.shape[1]):
            e = np.zeros_like(w64)
            e[i, j] = 0.5
            num[i, j] = (loss(w64 + e) - loss(w64 - e)) / 1.0
    assert np.allclose(dw, num, rtol=1e-12, atol=1e-12 * np.abs(num).max())


def test_dx_is_orthogonal_to_x_without_eps():
    """RMSNorm(a x) = RMSNorm(x) for a > 0 when eps = 0, so every derivative of it is
    orthogonal to x: sum_k x_k dx_k = 0 per row (a wrong sign or a dropped term breaks it)."""
    x, _, t, mu, dy, gain = _setup(5, 64, 7, 44, True)
    dx, _, _ = oracle.bitlinear_bwd(x, t, mu, dy, gain, 0.0)
    dots = np.sum(x.astype(np.float64) * dx, axis=1)
    assert np.all(np.abs(dots) <= 1e-12 * np.sum(np.abs(x * dx), axis=1))


def test_zero_upstream_gradient_gives_zero():
    x, _, t, mu, dy, gain = _setup(2, 16, 3, 45, True)
    dx, dw, dgain = oracle.bitlinear_bwd(x, t, mu, np.zeros_like(dy), gain)
    assert not dx.any() and not dw.any() and not dgain.any()
