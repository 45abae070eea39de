"""Pin for the oracle's block derivative: torch's reverse-mode differentiation (binary64, CPU)
of the block written with straight-through quantisers -- each quantised operand enters as
v + (v^ - v).detach(), so the forward value is the oracle's quantised one and the derivative
passes straight through -- must equal the oracle's hand-derived chain."""
import numpy as np
import pytest

import oracle
from ternary_weight_matmul_amd import synth

torch = pytest.importorskip("torch")


def _ste_linear(v, w_latent, lin, eps):
    """FusedBitLinear with straight-through quantisers, forward values from the oracle."""
    q, s, _ = oracle.quantize(v.detach().numpy(), lin.gain, eps)
    r = torch.rsqrt(torch.mean(v * v, dim=-1, keepdim=True) + float(np.float32(eps)))
    u = v * r
    if lin.gain is not None:
        u = u * lin.gain_t
    u_hat = torch.from_numpy(q.astype(np.float64) / s.astype(np.float64)[..., None])
    uq = u + (u_hat - u).detach()
    w_hat = torch.from_numpy(lin.t.astype(np.float64) / np.float64(oracle.weight_scale(lin.mu)))
    wq = w_latent + (w_hat - w_latent).detach()
    return uq @ wq.T


@pytest.mark.parametrize("gains", [None, "distinct"])
def test_block_derivative_matches_reverse_mode(gains):
    d, inner, b, t, eps = 32, 48, 2, 5, 1e-8
    lat = synth.latent_weights(d, inner, 61)
    gn = synth.norm_gains(d, inner, 62) if gains else None
    L = oracle.make_layer(lat, gn, eps)
    x = synth.activations((b, t, d), 63)
    h0 = synth.activations((b, d), 64)
    dout = synth.activations((b, t, d), 65)
    dhl = synth.activations((b, d), 66)
    ref = oracle.layer_backward(L, x, dout, h0, dhl)

    names = ("i", "f", "g", "o", "gate", "down")
    W = {k: torch.tensor(lat[k].astype(np.float64), requires_grad=True) for k in names}
    lins = {k: getattr(L, k) for k in names}
    G = {}
    for k in names:
        if lins[k].gain is not None:
            G[k] = torch.tensor(lins[k].gain.astype(np.float64), requires_grad=True)
            lins[k].gain_t = G[k]
    wn = torch.tensor(np.ones(d) if L.g_norm_w is None else L.g_norm_w.astype(np.float64), requires_grad=True)
    X = torch.tensor(x.astype(np.float64), requires_grad=True)
    H0 = torch.tensor(h0.astype(np.float64), requires_grad=True)

    ih = _ste_linear(X, W["i"], lins["i"], eps)
    fh = _ste_linear(X, W["f"], lins["f"], eps)
    gh = _ste_linear(X, W["g"], lins["g"], eps)
    f = torch.sigmoid(fh)
    xt = (1 - f) * torch.nn.functional.silu(ih)
    hs, state = [], H0
    for s_ in range(t):
        state = f[:, s_] * state + xt[:, s_]
        hs.append(state)
    h = torch.stack(hs, dim=1)
    rh = torch.rsqrt(torch.mean(h * h, dim=-1, keepdim=True) + float(np.float32(eps)))
    u = h * rh * wn * torch.nn.functional.silu(gh)
    x1 = X + _ste_linear(u, W["o"], lins["o"], eps)
    ab = _ste_linear(x1, W["gate"], lins["gate"], eps)
    z = torch.nn.functional.silu(ab[..., :inner]) * ab[..., inner:]
    out = x1 + _ste_linear(z, W["down"], lins["down"], eps)
    loss = torch.sum(out * torch.from_numpy(dout.astype(np.float64))) + \
        torch.sum(h[:, -1] * torch.from_numpy(dhl.astype(np.float64)))
    loss.backward()

    def close(a, b_, what):
        a, b_ = np.asarray(a, np.float64), np.asarray(b_, np.float64)
        assert np.max(np.abs(a - b_)) <= 1e-9 * (np.max(np.abs(b_)) + 1e-300), what

    close(ref["dx"], X.grad.numpy(), "dx")
    close(ref["dh0"], H0.grad.numpy(), "dh0")
    close(ref["dg_norm_w"], wn.grad.numpy(), "dg_norm_w")
    for k in names:
        close(ref["dw"][k], W[k].grad.numpy(), "dw " + k)
        if k in G:
            close(ref["dgain"][k], G[k].grad.numpy(), "dgain " + k)
