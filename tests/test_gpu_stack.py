"""GPU parity of the whole-stack decode step (mmf_stack_decode_step): one persistent kernel for
every block of a stack against (a) the chain of per-block decode steps, bit for bit, over
several steps with the states carried, and (b) the CPU oracle's own chain of blocks run free.
"""
import numpy as np
import pytest

import oracle
from ternary_weight_matmul_amd import synth
from parity import assert_close, bf16_tensor, dev, host, make_pair

pytestmark = pytest.mark.gpu


def _mmf():
    import ternary_weight_matmul_amd as mmf
    return mmf


def _stack(d, inner, n, seed, gpu, gains):
    pairs = [make_pair(d, inner, synth.layer_seed(seed, l), gpu, gains) for l in range(n)]
    return [p[0] for p in pairs], [p[1] for p in pairs]


def _act(a, act, gpu):
    return bf16_tensor(a, gpu) if act == "bf16" else dev(a, gpu)


@pytest.mark.parametrize("d,inner,n,b,act,gains,steps", [
    (1024, 2816, 3, 1, "f32", None, 2),
    (1024, 2816, 4, 5, "bf16", "shared", 2),
    (1024, 2816, 2, 16, "bf16", ("g_norm",), 3),
    (2048, 5632, 3, 16, "bf16", None, 3),
    (2048, 5632, 2, 16, "f32", "shared", 2),
    (2048, 5632, 2, 1, "bf16", None, 2),
    (2560, 6912, 2, 4, "bf16", None, 1),
])
def test_stack_step_equals_block_chain(gpu, d, inner, n, b, act, gains, steps):
    """The stack kernel's output and every block's state equal those of n mmf_layer_decode_step
    calls chained through buffers of the activation dtype, bit for bit, step after step."""
    import torch
    mmf = _mmf()
    _, P = _stack(d, inner, n, 2300 + d + n, gpu, gains)
    h0 = [synth.activations((b, d), 2400 + l) for l in range(n)]
    h_chain = [dev(h, gpu) for h in h0]
    h_stack = [dev(h, gpu) for h in h0]
    dec = mmf.StackDecoder(P, h_stack, b)
    for s in range(steps):
        x = _act(synth.activations((b, d), 2500 + 7 * s, act), act, gpu)
        cur = x
        for l in range(n):
            cur = mmf.layer_decode_step(P[l], cur, h_chain[l])
        out = dec.step(x)
        torch.cuda.synchronize()
        assert mmf.last_path() == "stack_decode;", mmf.last_path()
        assert out.dtype == x.dtype
        assert torch.equal(out, cur), (s, (out.float() - cur.float()).abs().max().item())
        for l in range(n):
            assert torch.equal(h_stack[l], h_chain[l]), (s, l)
    assert mmf.stack_decode_expired() == 0


def _oracle_chain(Ls, x, hs, act):
    """The oracle's blocks chained free: each block's output, rounded to the activation dtype
    (the type the entry points exchange between blocks), is the next block's input."""
    cur = x
    states = []
    for L, h in zip(Ls, hs):
        r = oracle.layer_decode_step(L, cur, h)
        states.append(r["h"])
        out = np.asarray(r["out"], np.float32)
        cur = synth.bf16_round(out) if act == "bf16" else out
    return cur, states


@pytest.mark.timeout(600)
@pytest.mark.parametrize("d,inner,n,b,act", [(1024, 2816, 4, 4, "f32"), (2048, 5632, 24, 16, "bf16")])
def test_stack_against_oracle_chain(gpu, d, inner, n, b, act):
    """The stack kernel against the oracle's own chain of blocks, run free: the first block's
    state within fp32 rounding (its only quantiser input is x, the same on both sides); every
    block's state and the output normwise, within a bound that grows with depth (a later
    quantiser's input differs by rounding, so a code may flip by one where its input lies
    within rounding of a decision point)."""
    mmf = _mmf()
    import torch
    Ls, P = _stack(d, inner, n, 2600 + n, gpu, None)
    h0 = [synth.activations((b, d), 2700 + l) for l in range(n)]
    hs = [dev(h, gpu) for h in h0]
    x = synth.activations((b, d), 2800, act)
    dec = mmf.StackDecoder(P, hs, b)
    out = dec.step(_act(x, act, gpu))
    torch.cuda.synchronize()
    ref_out, ref_h = _oracle_chain(Ls, x, h0, act)
    assert_close(host(hs[0]), ref_h[0], 1e-4, "state of block 0")
    base = 1e-3 if act == "f32" else 4e-3
    for l in range(n):
        hg = np.asarray(host(hs[l]), np.float64)
        rel = np.linalg.norm(hg - ref_h[l]) / np.linalg.norm(ref_h[l])
        assert rel < base * (1 + l), (l, rel)
    og = np.asarray(host(out), np.float64)
    rel = np.linalg.norm(og - ref_out) / np.linalg.norm(ref_out)
    assert rel < base * n, rel
    assert mmf.stack_decode_expired() == 0


def test_stack_rejects_and_reports(gpu):
    """Shapes the kernel does not take are refused before any launch, with a reason."""
    import torch
    mmf = _mmf()
    _, P = _stack(1024, 2816, 2, 2900, gpu, None)
    hs = [torch.zeros((17, 1024), dtype=torch.float32, device=gpu) for _ in range(2)]
    with pytest.raises(mmf.MMFError) as e:
        mmf.StackDecoder(P, hs, 17)
    assert e.value.status == 2 and "1..16" in str(e.value)
    _, Pd = _stack(1024, 2816, 1, 2901, gpu, "distinct")  # i, f and g each with their own gain
    with pytest.raises(mmf.MMFError) as e:
        mmf.StackDecoder(Pd, [torch.zeros((4, 1024), dtype=torch.float32, device=gpu)], 4)
    assert e.value.status == 2 and "gain" in str(e.value)


def test_stack_refuses_graph_capture(gpu):
    """A cooperative launch cannot be captured: on a capturing stream the call is refused before
    anything is enqueued, and the captured graph holds only the caller's own work."""
    import torch
    mmf = _mmf()
    _, P = _stack(1024, 2816, 2, 2950, gpu, None)
    h0 = [synth.activations((2, 1024), 2960 + l) for l in range(2)]
    hs = [dev(h, gpu) for h in h0]
    dec = mmf.StackDecoder(P, hs, 2)
    x = _act(synth.activations((2, 1024), 2970, "bf16"), "bf16", gpu)
    out = torch.zeros_like(x)
    y = torch.zeros(4, device=gpu)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    refused = None
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            y.add_(1.0)
            try:
                dec.step(x, out=out)
            except mmf.MMFError as e:
                refused = e
    assert refused is not None and refused.status == 2 and "captured" in str(refused)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(y, torch.ones(4, device=gpu))
    assert torch.equal(out, torch.zeros_like(x))
    for l in range(2):
        assert np.array_equal(host(hs[l]), h0[l])
    dec.step(x, out=out)  # outside capture it runs
    torch.cuda.synchronize()
    assert mmf.stack_decode_expired() == 0
