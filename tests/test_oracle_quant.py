"""Pins for the oracle's quantisers and ternary contraction.

Each test checks the oracle against something other than itself: hand-worked
values (tests/golden), exact ties, closed-form statistics of the Gaussian,
exact scale invariances and numpy's integer matrix product.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from ternary_weight_matmul_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def test_bitlinear_hand_worked():
    g = _golden("bitlinear_tiny.json")
    x = np.array(g["x"], np.float32)
    q, s, sq = oracle.quantize(x)
    assert q.tolist() == g["q"]
    assert sq.tolist() == g["sumq"]
    np.testing.assert_allclose(s, g["s"], rtol=1e-6)
    t, mu = oracle.ternarize(np.array(g["w"], np.float32))
    assert t.tolist() == g["t"]
    assert abs(float(mu) - g["mu"]) <= 1e-7 * g["mu"]
    r = oracle.bitlinear(x, t, mu)
    assert r["acc"].tolist() == g["acc"]
    np.testing.assert_allclose(r["y"], g["y"], rtol=2e-6)


def test_gain_applied_before_absmax():
    g = _golden("bitlinear_tiny.json")
    q, s, _ = oracle.quantize(np.array(g["x"], np.float32), gain=np.array(g["gain"], np.float32))
    assert q.tolist() == g["q_gain"]
    np.testing.assert_allclose(s, g["s_gain"], rtol=1e-5)


def test_ternary_ties_round_half_even():
    g = _golden("ternary_ties.json")
    t, mu = oracle.ternarize(np.array(g["w"], np.float32))
    assert float(mu) == g["mu"]
    assert t.tolist() == g["t"]


def test_gaussian_zero_fraction_closed_form():
    # P(t = 0) = P(|W| < E|W| / 2) = 2*Phi(sqrt(2/pi)/2) - 1 for Gaussian W, any sigma.
    w = synth.rng(11).standard_normal((512, 512), dtype=np.float32) * np.float32(0.02)
    t, mu = oracle.ternarize(w)
    p0 = math.erf(math.sqrt(2 / math.pi) / 2 / math.sqrt(2))
    assert abs(p0 - 0.3101) < 1e-4
    frac = float(np.mean(t == 0))
    assert abs(frac - p0) < 0.005          # ~5 binomial sigma
    assert abs(float(mu) - 0.02 * math.sqrt(2 / math.pi)) < 2e-4
    nz = t != 0
    assert np.all(np.sign(w[nz]) == t[nz])
    assert set(np.unique(t).tolist()) <= {-1, 0, 1}


def test_ternary_power_of_two_scale_invariance():
    w = synth.rng(12).standard_normal((64, 96), dtype=np.float32) * np.float32(0.02)
    t1, mu1 = oracle.ternarize(w)
    t2, mu2 = oracle.ternarize(w * np.float32(4.0))
    assert np.array_equal(t1, t2)
    assert float(mu2) == 4.0 * float(mu1)


def test_ternary_zero_tensor():
    t, mu = oracle.ternarize(np.zeros((3, 16), np.float32))
    assert float(mu) == 0.0 and not t.any()


def test_activation_quant_invariants():
    v = synth.rng(13).standard_normal((40, 160), dtype=np.float32) * np.float32(3.0)
    v[5] = 0.0
    q, s, sq = oracle.quantize(v)
    assert np.all(np.abs(q.astype(int)) <= 127)
    amax = np.abs(q.astype(int)).max(axis=1)
    assert np.all(amax[np.arange(40) != 5] == 127)
    assert not q[5].any() and sq[5] == 0
    assert np.array_equal(sq, q.astype(np.int64).sum(axis=1))
    nz = q != 0
    assert np.all(np.sign(v[nz]) == np.sign(q[nz]))
    # q/s approximates RMSNorm(v): its mean square is 1 up to the rounding of the codes.
    rows = np.arange(40) != 5
    ms = np.mean((q[rows].astype(np.float64) / s[rows, None]) ** 2, axis=1)
    assert np.all(np.abs(ms - 1.0) < 0.02)
    # the dequantised codes are within half a step of the normalised input
    y = v[rows] / np.sqrt(np.mean(v[rows].astype(np.float64) ** 2, axis=1, keepdims=True))
    err = np.abs(q[rows] / s[rows, None] - y)
    assert np.all(err <= 0.5 / s[rows, None] * (1 + 1e-5) + 1e-6)


def test_activation_quant_power_of_two_invariance():
    v = synth.rng(14).standard_normal((8, 64), dtype=np.float32)
    q1, s1, _ = oracle.quantize(v, eps=0.0)
    q2, s2, _ = oracle.quantize(v * np.float32(4.0), eps=0.0)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_ternary_matmul_matches_integer_matmul():
    g = synth.rng(15)
    q = g.integers(-128, 128, size=(7, 48), dtype=np.int8)
    t = g.integers(-1, 2, size=(13, 48), dtype=np.int8)
    acc = oracle.ternary_matmul(q, t)
    assert acc.shape == (7, 13)
    ref = q.astype(np.int64) @ t.astype(np.int64).T
    assert np.array_equal(acc, ref)
    # offset-code identity: sum (t+1)*q - sum q = sum t*q
    c = (t.astype(np.int64) + 1)
    assert np.array_equal(q.astype(np.int64) @ c.T - q.astype(np.int64).sum(1, keepdims=True), ref)


def test_ternary_matmul_extremes():
    k = 6912
    q = np.full((2, k), -128, np.int8)
    t = np.stack([np.ones(k, np.int8), -np.ones(k, np.int8)])
    acc = oracle.ternary_matmul(q, t)
    assert acc.tolist() == [[-128 * k, 128 * k], [-128 * k, 128 * k]]
    assert abs(128 * k) < 2 ** 24  # exact as float32 too


def test_pack_roundtrip_and_bit_layout():
    t = np.zeros((1, 32), np.int8)
    t[0, 0] = 1       # k=0  -> word 0, j=0, b=0: bits [0,2)  code 2
    t[0, 5] = -1      # k=5  -> word 0, j=1, b=1: bits [10,12) code 0
    t[0, 31] = 1      # k=31 -> word 1, j=3, b=3: bits [30,32) code 2
    w = oracle.pack(t)
    base = 0x55555555  # every code 1 (t = 0)
    assert w[0, 0] == (base & ~(3 << 0) | (2 << 0)) & ~(3 << 10)
    assert w[0, 1] == (base & ~(3 << 30)) | (2 << 30)
    g = synth.rng(16)
    tt = g.integers(-1, 2, size=(9, 80), dtype=np.int8)
    assert np.array_equal(oracle.unpack(oracle.pack(tt), 80), tt)
    # (word >> 2j) & 0x03030303 gives the codes of k = 16w+4j .. 16w+4j+3 in byte order
    words = oracle.pack(tt)
    for j in range(4):
        lanes = ((words[:, 0] >> (2 * j)) & 0x03030303).astype(np.uint32)
        by = lanes.view(np.uint8).reshape(9, 4).astype(int) - 1
        assert np.array_equal(by, tt[:, 4 * j:4 * j + 4])


def test_pack_rejects_bad_k():
    with pytest.raises(ValueError):
        oracle.pack(np.zeros((2, 20), np.int8))


def test_identity_weights_reproduce_normalised_input():
    k, c = 64, 0.37
    w = (np.eye(k) * c).astype(np.float32)
    t, mu = oracle.ternarize(w)
    assert np.array_equal(t, np.eye(k, dtype=np.int8))
    x = synth.rng(17).standard_normal((5, k), dtype=np.float32)
    r = oracle.bitlinear(x, t, mu)
    sw = float(oracle.weight_scale(mu))
    y = x / np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=1, keepdims=True))
    amax = np.abs(y).max(axis=1, keepdims=True)
    assert np.all(np.abs(r["y"] * sw - y) <= amax / 254 * (1 + 1e-4))
