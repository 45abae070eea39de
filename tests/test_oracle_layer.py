"""Pins for the oracle's HGRNBit block.

Special cases that remove the matrices (zero input, identity and zero
weights) reduce the block to short elementwise formulas written out here from
the definitions; they fail on a wrong gate wiring, a dropped (1 - f) factor,
a swapped MLP half or a missing residual. Structural properties (batch rows
independent, a sequence split in two with the state carried) hold at any size.
"""
import numpy as np

import oracle
from ternary_weight_matmul_amd import synth


def _layer(d, inner, seed, gains=False):
    lat = synth.latent_weights(d, inner, seed)
    gn = synth.norm_gains(d, inner, seed + 1) if gains else None
    return oracle.make_layer(lat, gn)


def test_zero_input_gives_zero_output():
    L = _layer(64, 96, 31)
    r = oracle.layer_forward(L, np.zeros((2, 5, 64)))
    assert not r["out"].any() and not r["h"].any()
    assert np.all(r["f"] == 0.5) and not r["xt"].any()


def test_identity_weight_block_closed_form():
    d, c, eps = 32, 0.25, 1e-8
    eye = (np.eye(d) * c).astype(np.float32)
    zero = np.zeros((d, d), np.float32)
    lat = {"i": eye, "f": zero, "g": eye, "o": eye,
           "gate": np.concatenate([eye, -eye]), "down": eye}
    L = oracle.make_layer(lat, eps=eps)
    x = synth.activations((1, 6, d), 32)
    r = oracle.layer_forward(L, x)

    def deq(v):  # identity ternary weights: the projection returns its quantised input / sw
        q, s, _ = oracle.quantize(v, None, eps)
        return q.astype(np.float64) / s.astype(np.float64)[..., None] * (c / d)

    ihat = deq(x)
    # f_proj has all-zero weights: f = sigmoid(0) = 1/2 exactly
    f = np.full_like(ihat, 0.5)
    xt = 0.5 * ihat / (1 + np.exp(-ihat))
    h = np.zeros_like(xt)
    for t in range(6):
        h[:, t] = xt[:, t] * 1.0 + (0.5 * h[:, t - 1] if t else 0.0)
    u = h / np.sqrt(np.mean(h ** 2, axis=-1, keepdims=True) + np.float64(np.float32(eps))) * ihat / (1 + np.exp(-ihat))
    x1 = x + deq(u)
    a = deq(x1)
    z = a / (1 + np.exp(-a)) * (-a)          # second half of gate_proj is -identity
    out = x1 + deq(z)
    np.testing.assert_allclose(r["f"], f, rtol=0, atol=0)
    np.testing.assert_allclose(r["h"], h, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["u"], u, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["x1"], x1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["z"], z, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["out"], out, rtol=1e-12, atol=1e-14)


def test_identity_weight_block_with_g_norm_gain():
    """The same closed form with a g_norm gain w: u = (h / rms(h)) * w * SiLU(g), the gain on the
    normalised state (not on g, not after o_proj's own normalisation)."""
    d, c, eps = 32, 0.25, 1e-8
    eye = (np.eye(d) * c).astype(np.float32)
    zero = np.zeros((d, d), np.float32)
    lat = {"i": eye, "f": zero, "g": eye, "o": eye, "gate": np.concatenate([eye, -eye]), "down": eye}
    w = (1.0 + 0.5 * np.sin(np.arange(d))).astype(np.float32)
    L = oracle.make_layer(lat, {"g_norm": w}, eps=eps)
    x = synth.activations((1, 5, d), 41)
    r = oracle.layer_forward(L, x)

    def deq(v):
        q, s, _ = oracle.quantize(v, None, eps)
        return q.astype(np.float64) / s.astype(np.float64)[..., None] * (c / d)

    ihat = deq(x)
    xt = 0.5 * ihat / (1 + np.exp(-ihat))
    h = np.zeros_like(xt)
    for t in range(5):
        h[:, t] = xt[:, t] + (0.5 * h[:, t - 1] if t else 0.0)
    rms = np.sqrt(np.mean(h ** 2, axis=-1, keepdims=True) + np.float64(np.float32(eps)))
    u = h / rms * w.astype(np.float64) * (ihat / (1 + np.exp(-ihat)))
    np.testing.assert_allclose(r["u"], u, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["x1"], x + deq(u), rtol=1e-12, atol=1e-14)


def test_batch_rows_independent():
    L = _layer(48, 64, 33, gains=True)
    x = synth.activations((3, 4, 48), 34)
    r = oracle.layer_forward(L, x)
    for b in range(3):
        rb = oracle.layer_forward(L, x[b:b + 1])
        assert np.array_equal(rb["out"][0], r["out"][b])


def test_split_sequence_equals_whole_and_decode_steps():
    L = _layer(48, 64, 35, gains=True)
    x = synth.activations((2, 7, 48), 36)
    h0 = synth.activations((2, 48), 37)
    r = oracle.layer_forward(L, x, h0)
    r1 = oracle.layer_forward(L, x[:, :3], h0)
    r2 = oracle.layer_forward(L, x[:, 3:], r1["h_last"])
    assert np.array_equal(np.concatenate([r1["out"], r2["out"]], 1), r["out"])
    h = h0.astype(np.float64)
    for t in range(7):
        st = oracle.layer_decode_step(L, x[:, t], h)
        assert np.array_equal(st["out"], r["out"][:, t])
        h = st["h"]
    assert np.array_equal(h, r["h_last"])


def test_stage_shapes_and_codes():
    L = _layer(64, 96, 38)
    x = synth.activations((2, 3, 64), 39)
    r = oracle.layer_forward(L, x)
    assert r["out"].shape == (2, 3, 64) and r["z"].shape == (2, 3, 96)
    assert r["acc_gate"].shape == (2, 3, 192)
    for k in ("q_i", "q_u", "q_x1", "q_z"):
        assert r[k].dtype == np.int8
    # i/f/g share one quantisation of x when their gains are equal
    assert np.array_equal(r["q_i"], r["q_f"]) and np.array_equal(r["q_i"], r["q_g"])


# ---------------------------------------------------------------------------
# Gate orientation at the mixer level: f = sigmoid(f_proj) is the forget gate
# of h_t = f_t h_{t-1} + x~_t ("MatMul-Free LLM 深度分析报告", table 创新之处) and
# x~ = (1 - f) SiLU(i_proj) its input. Identity i/g weights and f_proj = -C I or
# +C I (C large) drive f_proj's output to about -/+5000 on every channel of an
# all-positive input, where sigmoid is exactly 0 or 1 in binary64.
# ---------------------------------------------------------------------------

def _saturated_gate_block(sign, d=32, c=0.25, big=1e4, eps=1e-8):
    eye = (np.eye(d) * c).astype(np.float32)
    f_w = (np.eye(d) * (sign * big * d)).astype(np.float32)  # mean |W| = big
    lat = {"i": eye, "f": f_w, "g": eye, "o": eye, "gate": np.concatenate([eye, -eye]), "down": eye}
    L = oracle.make_layer(lat, eps=eps)
    x = (1.0 + synth.rng(51).random((2, 6, d))).astype(np.float32)  # all in [1, 2)
    return L, x, c / d


def _deq(v, scale, eps=1e-8):
    q, s, _ = oracle.quantize(v, None, eps)
    return q.astype(np.float64) / s.astype(np.float64)[..., None] * scale


def _check_forget_gate_zero(L, x, scale, h0):
    """f == 0: the mixer is a per-token gated feed-forward, h_t = x~_t = SiLU(i^_t)."""
    with np.errstate(over="ignore"):
        r = oracle.layer_forward(L, x, h0)
    assert np.all(r["f_hat"] < -800)
    assert np.all(r["f"] == 0.0)
    ihat = _deq(x, scale)
    silu_i = ihat / (1 + np.exp(-ihat))
    np.testing.assert_allclose(r["xt"], silu_i, rtol=1e-13, atol=0)
    np.testing.assert_allclose(r["h"], silu_i, rtol=1e-13, atol=0)  # no carry from h0 or earlier tokens
    # tokens are independent: a permutation of the tokens permutes the outputs
    perm = np.array([3, 0, 5, 1, 4, 2])
    with np.errstate(over="ignore"):
        rp = oracle.layer_forward(L, x[:, perm], None)
    assert np.array_equal(rp["out"], r["out"][:, perm])
    assert np.array_equal(rp["h"], r["h"][:, perm])


def _check_forget_gate_one(L, x, scale, h0):
    """f == 1: x~ = 0 and the state never moves, h_t = h_0 for every t."""
    r = oracle.layer_forward(L, x, h0)
    assert np.all(r["f_hat"] > 800)
    assert np.all(r["f"] == 1.0)
    assert not r["xt"].any()
    assert np.array_equal(r["h"], np.broadcast_to(h0[:, None, :], r["h"].shape))
    ghat = _deq(x, scale)
    rms = np.sqrt(np.mean(h0 ** 2, axis=-1, keepdims=True) + np.float64(np.float32(1e-8)))
    u = (h0 / rms)[:, None, :] * (ghat / (1 + np.exp(-ghat)))
    np.testing.assert_allclose(r["u"], u, rtol=1e-12, atol=1e-14)


def test_forget_gate_zero_makes_the_mixer_a_gated_feed_forward():
    L, x, scale = _saturated_gate_block(-1)
    h0 = synth.activations((2, 32), 52).astype(np.float64)
    _check_forget_gate_zero(L, x, scale, h0)


def test_forget_gate_one_holds_the_state():
    L, x, scale = _saturated_gate_block(+1)
    h0 = synth.activations((2, 32), 53).astype(np.float64)
    _check_forget_gate_one(L, x, scale, h0)


def _swapped(f_hat_i, f_hat_f):  # planted mistake: f and 1 - f exchanged
    f = oracle.sigmoid(f_hat_f)
    return 1.0 - f, f * oracle.silu(f_hat_i)


def _negated(f_hat_i, f_hat_f):  # planted mistake: sigmoid of -f_proj
    f = oracle.sigmoid(-np.asarray(f_hat_f, np.float64))
    return f, (1.0 - f) * oracle.silu(f_hat_i)


def _inverted_input(f_hat_i, f_hat_f):  # planted mistake: x~ = f SiLU(i) with the forget gate kept
    f = oracle.sigmoid(f_hat_f)
    return f, f * oracle.silu(f_hat_i)


def test_gate_orientation_pins_catch_planted_mistakes(monkeypatch):
    """Each planted orientation mistake in a copy of the gates fails both pins above."""
    import pytest
    h0 = synth.activations((2, 32), 54).astype(np.float64)
    for planted in (_swapped, _negated, _inverted_input):
        monkeypatch.setattr(oracle, "mixer_gates", planted)
        failed = 0
        for sign, check in ((-1, _check_forget_gate_zero), (+1, _check_forget_gate_one)):
            L, x, scale = _saturated_gate_block(sign)
            try:
                with np.errstate(over="ignore", invalid="ignore"):
                    check(L, x, scale, h0)
            except AssertionError:
                failed += 1
        assert failed == 2, planted.__name__
        monkeypatch.undo()
