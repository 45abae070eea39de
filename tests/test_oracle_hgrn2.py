"""Pins for the oracle's expanded-state recurrence (``oracle.hgrn2_scan``).

The recurrence is [R1]'s h_t = g_t * h_{t-1} + x_t ("MatMul-Free LLM 深度分析报告",
section "核心价值提炼", table "创新之处") with each head's state widened to an e x e matrix:
S_t = diag(f_t) S_{t-1} + (1 - f_t) i_t^T, y_t = S_t^T o_t. Its equations are not printed on the
pages (a reading); these pins fix the reading's own consequences from outside the function:
the unrolled sum in exact rationals, the e = 1 case against the elementwise recurrence, the
saturated gates, head independence, the carried state and linearity. A copy of the function
with a plausible mistake planted in it fails the exact pin.
"""
from fractions import Fraction

import numpy as np

import oracle
from ternary_weight_matmul_amd import synth


def _dyadic(g, shape, den, lo, hi):
    """Exact small dyadic rationals k / den with k in [lo, hi]."""
    return g.integers(lo, hi + 1, size=shape) / den


def _exact_unrolled(f, i, o, e, s0):
    """y_t and S_t from the unrolled sum, in exact rationals:
    S_t[a][c] = (prod_{r<=t} f_r[a]) S_0[a][c] + sum_{s<=t} (prod_{s<r<=t} f_r[a]) (1 - f_s[a]) i_s[c],
    y_t[c] = sum_a o_t[a] S_t[a][c]."""
    b, t, d = f.shape
    nh = d // e
    F = lambda v: Fraction(float(v))
    y = np.empty((b, t, d), dtype=object)
    s_last = np.empty((b, nh, e, e), dtype=object)
    for bb in range(b):
        for n in range(nh):
            ch = slice(n * e, (n + 1) * e)
            fb, ib, ob = f[bb, :, ch], i[bb, :, ch], o[bb, :, ch]
            for tt in range(t):
                S = [[None] * e for _ in range(e)]
                for a in range(e):
                    for c in range(e):
                        decay_all = Fraction(1)
                        for r in range(tt + 1):
                            decay_all *= F(fb[r, a])
                        acc = decay_all * F(s0[bb, n, a, c])
                        for s_ in range(tt + 1):
                            dec = Fraction(1)
                            for r in range(s_ + 1, tt + 1):
                                dec *= F(fb[r, a])
                            acc += dec * (1 - F(fb[s_, a])) * F(ib[s_, c])
                        S[a][c] = acc
                for c in range(e):
                    y[bb, tt, n * e + c] = sum((F(ob[tt, a]) * S[a][c] for a in range(e)), Fraction(0))
                if tt == t - 1:
                    for a in range(e):
                        for c in range(e):
                            s_last[bb, n, a, c] = S[a][c]
    return y, s_last


def _small_exact_case(seed=71, b=2, t=4, e=3, nh=2):
    g = synth.rng(seed)
    d = e * nh
    f = _dyadic(g, (b, t, d), 8, 1, 7)      # f in (0, 1)
    i = _dyadic(g, (b, t, d), 4, -8, 8)
    o = _dyadic(g, (b, t, d), 4, -8, 8)
    s0 = _dyadic(g, (b, nh, e, e), 4, -8, 8)
    return f, i, o, e, s0


def _check_exact(scan):
    f, i, o, e, s0 = _small_exact_case()
    y, s_last = scan(f, i, o, e, s0)
    ye, se = _exact_unrolled(f, i, o, e, s0)
    # dyadic inputs with small denominators: every binary64 step is exact
    assert np.array_equal(np.asarray(y, np.float64), ye.astype(np.float64)), "y differs from the unrolled sum"
    assert all(Fraction(float(v)) == w for v, w in zip(np.asarray(y).ravel(), ye.ravel()))
    assert np.array_equal(np.asarray(s_last, np.float64), se.astype(np.float64)), "state differs"


def test_exact_unrolled_sum():
    _check_exact(oracle.hgrn2_scan)


def test_head_width_one_is_the_elementwise_recurrence():
    """e = 1: S_t = f_t S_{t-1} + (1 - f_t) i_t is [R1]'s recurrence with x~ = (1 - f) i; y = o * h."""
    f, i, o = synth.hgrn2_inputs(2, 37, 8, 72)
    h0 = synth.activations((2, 8), 73)
    y, s_last = oracle.hgrn2_scan(f, i, o, 1, h0.reshape(2, 8, 1, 1))
    x = (1.0 - f.astype(np.float64)) * i.astype(np.float64)
    h = oracle.hgrn_scan(x, f, h0)
    np.testing.assert_allclose(y, o.astype(np.float64) * h, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(s_last.reshape(2, 8), h[:, -1], rtol=1e-13, atol=1e-14)


def test_forget_gate_zero_reads_out_the_current_input():
    """f == 0: S_t = 1 i_t^T (every row is i_t), so y_t = (sum_a o_t[a]) i_t with no history."""
    _, i, o = synth.hgrn2_inputs(2, 6, 16, 74)
    f = np.zeros_like(i)
    s0 = synth.activations((2, 2, 8, 8), 75)
    y, s_last = oracle.hgrn2_scan(f, i, o, 8, s0)
    oh = o.astype(np.float64).reshape(2, 6, 2, 8)
    ih = i.astype(np.float64).reshape(2, 6, 2, 8)
    want = oh.sum(-1, keepdims=True) * ih
    np.testing.assert_allclose(y, want.reshape(2, 6, 16), rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(s_last, np.broadcast_to(ih[:, -1][:, :, None, :], s_last.shape))
    perm = np.array([4, 0, 5, 2, 1, 3])
    yp, _ = oracle.hgrn2_scan(f[:, perm], i[:, perm], o[:, perm], 8, s0)
    assert np.array_equal(yp, y[:, perm])


def test_forget_gate_one_holds_the_state():
    """f == 1: the input term vanishes, S_t = S_0 and y_t = S_0^T o_t."""
    _, i, o = synth.hgrn2_inputs(2, 5, 16, 76)
    f = np.ones_like(i)
    s0 = synth.activations((2, 2, 8, 8), 77).astype(np.float64)
    y, s_last = oracle.hgrn2_scan(f, i, o, 8, s0)
    np.testing.assert_array_equal(s_last, s0)
    oh = o.astype(np.float64).reshape(2, 5, 2, 8)
    want = np.einsum("btna,bnac->btnc", oh, s0).reshape(2, 5, 16)
    np.testing.assert_allclose(y, want, rtol=1e-13, atol=1e-13)


def test_heads_are_independent():
    f, i, o = synth.hgrn2_inputs(2, 9, 32, 78)
    s0 = synth.activations((2, 4, 8, 8), 79)
    y, s = oracle.hgrn2_scan(f, i, o, 8, s0)
    perm = np.array([2, 0, 3, 1])
    cols = (perm[:, None] * 8 + np.arange(8)[None, :]).ravel()
    yp, sp = oracle.hgrn2_scan(f[..., cols], i[..., cols], o[..., cols], 8, s0[:, perm])
    assert np.array_equal(yp, y[..., cols])
    assert np.array_equal(sp, s[:, perm])


def test_carried_state_splits_the_sequence():
    f, i, o = synth.hgrn2_inputs(2, 11, 32, 80)
    s0 = synth.activations((2, 2, 16, 16), 81)
    y, s = oracle.hgrn2_scan(f, i, o, 16, s0)
    y1, s1 = oracle.hgrn2_scan(f[:, :4], i[:, :4], o[:, :4], 16, s0)
    y2, s2 = oracle.hgrn2_scan(f[:, 4:], i[:, 4:], o[:, 4:], 16, s1)
    assert np.array_equal(np.concatenate([y1, y2], 1), y) and np.array_equal(s2, s)
    st = s0
    for k in range(11):
        yk, st = oracle.hgrn2_scan(f[:, k:k + 1], i[:, k:k + 1], o[:, k:k + 1], 16, st)
        assert np.array_equal(yk[:, 0], y[:, k])
    assert np.array_equal(st, s)
    y0, s_empty = oracle.hgrn2_scan(f[:, :0], i[:, :0], o[:, :0], 16, s0)
    assert y0.shape == (2, 0, 32) and np.array_equal(s_empty, s0)


def test_linear_in_input_and_initial_state():
    """For fixed gates, (i, S_0) -> y is linear."""
    f, i1, o = synth.hgrn2_inputs(1, 7, 16, 82)
    _, i2, _ = synth.hgrn2_inputs(1, 7, 16, 83)
    a0 = synth.activations((1, 2, 8, 8), 84).astype(np.float64)
    b0 = synth.activations((1, 2, 8, 8), 85).astype(np.float64)
    ya, sa = oracle.hgrn2_scan(f, i1, o, 8, a0)
    yb, sb = oracle.hgrn2_scan(f, i2, o, 8, b0)
    yc, sc = oracle.hgrn2_scan(f, 2.0 * i1.astype(np.float64) - 3.0 * i2.astype(np.float64), o, 8, 2.0 * a0 - 3.0 * b0)
    np.testing.assert_allclose(yc, 2.0 * ya - 3.0 * yb, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sc, 2.0 * sa - 3.0 * sb, rtol=1e-12, atol=1e-12)


# planted mistakes, each in a copy of the recurrence

def _scan_variant(kind):
    def scan(f, i, o, e, s0):
        b, t, d = f.shape
        nh = d // e
        fh = np.asarray(f, np.float64).reshape(b, t, nh, e)
        ih = np.asarray(i, np.float64).reshape(b, t, nh, e)
        oh = np.asarray(o, np.float64).reshape(b, t, nh, e)
        s = np.array(s0, np.float64).reshape(b, nh, e, e)
        y = np.empty((b, t, nh, e))
        for k in range(t):
            fr = fh[:, k][..., :, None]
            fc = fh[:, k][..., None, :]
            prev = s
            if kind == "gate_on_columns":
                s = fc * s + (1.0 - fc) * ih[:, k][..., None, :]
            elif kind == "unscaled_input":
                s = fr * s + ih[:, k][..., None, :]
            else:
                s = fr * s + (1.0 - fr) * ih[:, k][..., None, :]
            read = prev if kind == "reads_previous_state" else s
            if kind == "transposed_readout":
                y[:, k] = np.einsum("bnc,bnac->bna", oh[:, k], read)
            else:
                y[:, k] = np.einsum("bna,bnac->bnc", oh[:, k], read)
        return y.reshape(b, t, d), s
    return scan


def test_exact_pin_catches_planted_mistakes():
    _check_exact(_scan_variant("none"))  # the unplanted copy passes
    for kind in ("gate_on_columns", "unscaled_input", "reads_previous_state", "transposed_readout"):
        try:
            _check_exact(_scan_variant(kind))
        except AssertionError:
            continue
        raise AssertionError("planted mistake not caught: " + kind)
