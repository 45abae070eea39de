"""GPU parity: every C-ABI entry point against the CPU oracle on seeded inputs.

Sizes span several MFMA tiles with ragged tails (m, n, k not multiples of
the tile), the decode (m <= 64) and prefill (m > 64) contraction paths, both
scan modes, both activation dtypes and the three RMSNorm-gain layouts.
"""
import numpy as np
import pytest

import oracle
from ternary_weight_matmul_amd import synth
from parity import (assert_close, assert_equal, bf16_tensor, check_free_running, check_layer_sampled,
                    check_layer_stages, dev, host, make_pair, packed_words)

pytestmark = pytest.mark.gpu


def _mmf():
    import ternary_weight_matmul_amd as mmf
    return mmf


@pytest.mark.parametrize("n,k", [(1, 16), (7, 48), (130, 80), (64, 1024), (2048, 2048), (333, 2816)])
def test_pack_bit_exact(gpu, n, k):
    mmf = _mmf()
    w = synth.rng(100 + n + k).standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    t, mu = oracle.ternarize(w)
    pl = mmf.ternary_pack(dev(w, gpu))
    assert host(pl.mu)[0] == mu
    assert_equal(packed_words(pl), oracle.pack(t), "packed words")
    assert "pack" in mmf.last_path()


def test_pack_ties_round_half_even(gpu):
    mmf = _mmf()
    w = np.tile(np.array([0.5, -0.5, 1.5, -1.5], np.float32), (3, 4))
    t, mu = oracle.ternarize(w)
    assert mu == 1.0
    pl = mmf.ternary_pack(dev(w, gpu))
    assert_equal(packed_words(pl), oracle.pack(t), "tie words")


BITLINEAR_CASES = [
    # m, k, n, dtype, gain
    (1, 16, 1, "f32", False),
    (5, 48, 17, "f32", True),
    (16, 256, 64, "bf16", False),
    (64, 1040, 130, "f32", True),
    (49, 16, 40, "f32", False),        # four row blocks with a single K word
    (65, 80, 33, "f32", False),
    (200, 1024, 200, "bf16", True),
    (300, 2816, 96, "f32", False),
    (513, 2048, 1111, "bf16", False),
    # decode GEMV paths: two slices per wave (21 slices over 16 waves), two and four
    # channel blocks per workgroup (ragged last block), the double-buffered slice loop
    # (64 slices) and a K that is no whole number of slices (33 slices, last one partial)
    (3, 5376, 300, "bf16", True),
    (16, 2048, 5136, "f32", False),
    (8, 2048, 10250, "bf16", False),
    (16, 16384, 64, "bf16", False),
    (2, 8208, 100, "f32", True),
    # eight channel blocks per workgroup (single group, 20480 outputs or more), ragged last block;
    # with more slices than its eight waves, the double-buffered slice loop (32 slices; 17 with
    # the last one partial)
    (4, 1024, 20500, "bf16", True),
    (16, 2048, 32768, "f32", False),
    (16, 8192, 20480, "f32", False),
    (5, 4112, 20496, "bf16", True),
    # rows longer than 8192 at few rows: a 1024-thread quantiser workgroup per row
    (3, 12288, 40, "f32", True),
    (2, 9008, 24, "bf16", True),
]


@pytest.mark.parametrize("m,k,n,dt,with_gain", BITLINEAR_CASES)
def test_bitlinear_parity(gpu, m, k, n, dt, with_gain):
    import torch
    mmf = _mmf()
    g = synth.rng(200 + m + k + n)
    x = synth.activations((m, k), 300 + m, dt, std=2.0)
    w = (g.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    gain = (1 + 0.1 * g.standard_normal(k)).astype(np.float32) if with_gain else None
    t, mu = oracle.ternarize(w)
    pl = mmf.ternary_pack(dev(w, gpu), dev(gain, gpu) if gain is not None else None)
    xd = bf16_tensor(x, gpu) if dt == "bf16" else dev(x, gpu)
    codes = torch.empty((m, k), dtype=torch.int8, device=gpu)
    scale = torch.empty(m, dtype=torch.float32, device=gpu)
    acc = torch.empty((m, n), dtype=torch.int32, device=gpu)
    y = mmf.bitlinear_fwd(xd, pl, 1e-8, torch.float32, codes, scale, acc)
    torch.cuda.synchronize()
    path = mmf.last_path()
    assert ("tgemv" if m <= 64 else "tgemm") in path, path
    q, s, _ = oracle.quantize(x, gain)
    assert_equal(host(codes), q, "codes")
    assert_equal(host(scale), s, "scale")
    ref_acc = oracle.ternary_matmul(q, t)
    assert_equal(host(acc), ref_acc, "acc")
    assert_close(host(y), oracle.dequant(ref_acc, s, mu), 1e-4, "y")
    # the same call with bf16 output and no optional outputs
    yb = mmf.bitlinear_fwd(xd, pl, 1e-8, torch.bfloat16)
    assert_close(host(yb), oracle.dequant(ref_acc, s, mu), 2e-2, "y bf16")


def test_bitlinear_zero_rows_and_empty(gpu):
    import torch
    mmf = _mmf()
    x = synth.activations((70, 64), 7)
    x[3] = 0.0
    x[69] = 0.0
    w = synth.rng(8).standard_normal((32, 64), dtype=np.float32) * np.float32(0.02)
    pl = mmf.ternary_pack(dev(w, gpu))
    y = host(mmf.bitlinear_fwd(dev(x, gpu), pl))
    assert not y[3].any() and not y[69].any()
    empty = mmf.bitlinear_fwd(torch.empty((0, 64), device=gpu), pl)
    assert empty.shape == (0, 32)


SCAN_CASES = [
    # b, t, d, mode, with_h0
    (1, 1, 64, "recurrent", False),
    (2, 7, 48, "recurrent", True),
    (3, 300, 96, "recurrent", True),
    (2, 300, 96, "chunk", True),
    (1, 4099, 128, "chunk", False),
    (4, 2048, 256, "auto", True),
    # enough (sequence, 64-channel) groups for the single-pass tiled kernel:
    (8, 700, 1024, "chunk", True),     # ragged last chunk
    (16, 300, 520, "auto", False),     # partial channel group
    (2, 4100, 4096, "chunk", True),    # T >= 4096, streaming accesses
    (16, 260, 2048, "chunk", True),    # many groups: 4-wave workgroups, ragged last chunk
]


@pytest.mark.parametrize("b,t,d,mode,with_h0", SCAN_CASES)
def test_scan_parity(gpu, b, t, d, mode, with_h0):
    import torch
    mmf = _mmf()
    x, f = synth.scan_inputs(b, t, d, 400 + t + d)
    h0 = synth.activations((b, d), 401) if with_h0 else None
    h_last = torch.empty((b, d), device=gpu)
    h = mmf.hgrn_scan_fwd(dev(x, gpu), dev(f, gpu), dev(h0, gpu) if with_h0 else None, mode, h_last=h_last)
    ref = oracle.hgrn_scan(x, f, h0)
    rtol = 1e-3 if (mode != "recurrent" and t >= 4096) else 1e-4
    assert_close(host(h), ref, rtol, "h")
    assert_close(host(h_last), ref[:, -1], rtol, "h_last")
    if mode == "recurrent":
        assert "scan_recurrent" in mmf.last_path()
    elif b * ((d + 63) // 64) >= 128:
        assert "scan_tiled" in mmf.last_path()


def test_scan_in_place_and_empty(gpu):
    import torch
    mmf = _mmf()
    x, f = synth.scan_inputs(2, 500, 64, 402)
    ref = oracle.hgrn_scan(x, f)
    for mode in ("recurrent", "chunk"):
        xd = dev(x, gpu)
        h = mmf.hgrn_scan_fwd(xd, dev(f, gpu), None, mode, out=xd)
        assert h.data_ptr() == xd.data_ptr()
        assert_close(host(h), ref, 1e-4, "in-place " + mode)
    h0 = dev(synth.activations((2, 64), 403), gpu)
    h_last = torch.zeros((2, 64), device=gpu)
    mmf.hgrn_scan_fwd(torch.empty((2, 0, 64), device=gpu), torch.empty((2, 0, 64), device=gpu), h0, h_last=h_last)
    assert torch.equal(h_last, h0)


def test_scan_tiled_in_place(gpu):
    mmf = _mmf()
    x, f = synth.scan_inputs(4, 390, 2048, 405)
    h0 = synth.activations((4, 2048), 406)
    ref = oracle.hgrn_scan(x, f, h0)
    xd = dev(x, gpu)
    h = mmf.hgrn_scan_fwd(xd, dev(f, gpu), dev(h0, gpu), "chunk", out=xd)
    assert "scan_tiled" in mmf.last_path()
    assert h.data_ptr() == xd.data_ptr()
    assert_close(host(h), ref, 1e-4, "tiled in place")


def test_scan_c5_full_size_sampled(gpu):
    """The long-sequence stress shape: B=16, T=32768, d=2048, f = sigmoid(N(2,1)), chunked,
    in the configuration the layer uses. Each sequence is generated with its own seed; the
    oracle runs the whole sequence for 64 sampled channels (4 per sequence)."""
    import torch
    mmf = _mmf()
    b, t, d = 16, 32768, 2048
    xd = torch.empty((b, t, d), device=gpu)
    fd = torch.empty((b, t, d), device=gpu)
    pick = np.stack([synth.rng(5500 + i).choice(d, size=4, replace=False) for i in range(b)])
    xs, fs = [], []
    for i in range(b):
        x, f = synth.scan_inputs(1, t, d, 5 * 1000 + i)
        xd[i].copy_(torch.from_numpy(x[0]))
        fd[i].copy_(torch.from_numpy(f[0]))
        xs.append(x[0][:, pick[i]].copy())
        fs.append(f[0][:, pick[i]].copy())
        del x, f
    h_last = torch.empty((b, d), device=gpu)
    h = mmf.hgrn_scan_fwd(xd, fd, None, "chunk", h_last=h_last)
    assert "scan_tiled" in mmf.last_path()
    idx = torch.from_numpy(pick).to(gpu)
    got = torch.gather(h, 2, idx[:, None, :].expand(b, t, 4)).cpu().numpy()
    got_last = torch.gather(h_last, 1, idx).cpu().numpy()
    ref = oracle.hgrn_scan(np.stack(xs), np.stack(fs))
    assert_close(got, ref, 1e-3, "h (sampled channels)")
    assert_close(got_last, ref[:, -1], 1e-3, "h_last (sampled channels)")


def test_scan_limits_zero_and_unit_gate(gpu):
    mmf = _mmf()
    x = synth.activations((2, 257, 64), 404)
    xd = dev(x, gpu)
    h = host(mmf.hgrn_scan_fwd(xd, dev(np.zeros_like(x), gpu), None, "chunk"))
    assert np.array_equal(h, x)
    h = host(mmf.hgrn_scan_fwd(xd, dev(np.ones_like(x), gpu), None, "recurrent"))
    assert_close(h, np.cumsum(x.astype(np.float64), axis=1), 1e-5, "cumsum")


BITLINEAR_BWD_CASES = [
    # m, k, n, x dtype, dy dtype, with gain
    (3, 64, 32, "f32", "f32", False),
    (17, 256, 96, "bf16", "bf16", True),
    (64, 1024, 200, "f32", "bf16", True),
    (300, 512, 1024, "bf16", "bf16", False),
    (1000, 2048, 2048, "bf16", "f32", True),   # the 1.3B width
    (129, 5632, 2048, "bf16", "bf16", False),  # down_proj's shape, ragged row count
]


@pytest.mark.parametrize("m,k,n,xt,dyt,with_gain", BITLINEAR_BWD_CASES)
def test_bitlinear_bwd_parity(gpu, m, k, n, xt, dyt, with_gain):
    """dx, dW and dgain against the oracle's straight-through derivative. With a bf16 dy the
    first product is exact up to fp32 summation order (rtol 1e-4); an fp32 dy and the scaled
    codes of dW are rounded to bf16 on the way into the products (the bf16 bar, rtol 2e-2)."""
    import torch
    mmf = _mmf()
    x = synth.activations((m, k), 800 + m, xt)
    w = synth.rng(801 + k).standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    dy = synth.activations((m, n), 802 + n, dyt)
    gain = (1.0 + 0.1 * synth.rng(803).standard_normal(k)).astype(np.float32) if with_gain else None
    t, mu = oracle.ternarize(w)
    rdx, rdw, rdg = oracle.bitlinear_bwd(x, t, mu, dy, gain)
    pl = mmf.ternary_pack(dev(w, gpu), norm_w=dev(gain, gpu) if with_gain else None)
    xd = bf16_tensor(x, gpu) if xt == "bf16" else dev(x, gpu)
    dyd = bf16_tensor(dy, gpu) if dyt == "bf16" else dev(dy, gpu)
    dx, dw, dg = mmf.bitlinear_bwd(xd, pl, dyd, want_dgain=True, dx_dtype=torch.float32)
    torch.cuda.synchronize()
    tight = 1e-4 if dyt == "bf16" else 2e-2
    assert_close(host(dx), rdx, tight, "dx")
    assert_close(host(dg), rdg, tight, "dgain")
    assert_close(host(dw), rdw, 2e-2, "dw")
    assert "gemm_bf16<du>" in mmf.last_path() and "gemm_bf16<dw>" in mmf.last_path()


def test_bitlinear_bwd_outputs_optional_and_empty(gpu):
    import torch
    mmf = _mmf()
    m, k, n = 40, 256, 64
    x = synth.activations((m, k), 810, "bf16")
    w = synth.rng(811).standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    dy = synth.activations((m, n), 812, "bf16")
    t, mu = oracle.ternarize(w)
    rdx, rdw, _ = oracle.bitlinear_bwd(x, t, mu, dy)
    pl = mmf.ternary_pack(dev(w, gpu))
    xd, dyd = bf16_tensor(x, gpu), bf16_tensor(dy, gpu)
    dx, dw, dg = mmf.bitlinear_bwd(xd, pl, dyd, want_dw=False)
    assert dw is None and dg is None and dx.dtype == torch.bfloat16
    assert "gemm_bf16<dw>" not in mmf.last_path()
    assert_close(host(dx), rdx, 2e-2, "dx (bf16)")
    dx, dw, _ = mmf.bitlinear_bwd(xd, pl, dyd, want_dx=False)
    assert dx is None and "gemm_bf16<du>" not in mmf.last_path()
    assert_close(host(dw), rdw, 2e-2, "dw alone")
    # no rows: dW and dgain are empty sums
    _, dw, dg = mmf.bitlinear_bwd(torch.empty((0, k), device=gpu), pl, torch.empty((0, n), device=gpu),
                                  want_dgain=True)
    assert not host(dw).any() and not host(dg).any()


def test_embed_rows(gpu):
    import torch
    mmf = _mmf()
    for dtype in ("f32", "bf16"):
        table = synth.activations((1000, 272), 820, dtype)
        ids = np.array([5, 0, 999, -1, 1000, 5, 123], dtype=np.int32)
        td = bf16_tensor(table, gpu) if dtype == "bf16" else dev(table, gpu)
        out = mmf.embed(dev(ids, gpu), td)
        assert_equal(host(out), oracle.embed(ids, table), "embed " + dtype)
    assert mmf.embed(torch.empty((0,), dtype=torch.int32, device=gpu), td).shape == (0, 272)


GREEDY_CASES = [
    # b, k, vocab, x dtype, with gain
    (1, 2048, 32000, "bf16", False),   # the 1.3B head: width 2048, 32000 tokens
    (16, 2048, 32000, "bf16", True),
    (5, 256, 1000, "f32", False),
    (70, 512, 4096, "bf16", False),    # above the GEMV limit: tiled contraction
]


@pytest.mark.parametrize("b,k,vocab,xt,with_gain", GREEDY_CASES)
def test_greedy_head_parity(gpu, b, k, vocab, xt, with_gain):
    """Tokens bit-exact (the first largest exact sum); logits within the fp32 tolerance."""
    import torch
    mmf = _mmf()
    x = synth.activations((b, k), 830 + b, xt)
    w = synth.rng(831 + vocab).standard_normal((vocab, k), dtype=np.float32) * np.float32(0.02)
    gain = (1.0 + 0.1 * synth.rng(832).standard_normal(k)).astype(np.float32) if with_gain else None
    t, mu = oracle.ternarize(w)
    ref = oracle.greedy_head(x, t, mu, gain)
    pl = mmf.ternary_pack(dev(w, gpu), norm_w=dev(gain, gpu) if with_gain else None)
    xd = bf16_tensor(x, gpu) if xt == "bf16" else dev(x, gpu)
    logits = torch.empty((b, vocab), device=gpu)
    tokens = mmf.greedy_head(xd, pl, logits=logits)
    assert_equal(host(tokens), ref["tokens"], "tokens")
    assert_close(host(logits), ref["y"], 1e-4, "logits")
    assert "argmax_rows" in mmf.last_path()


def test_greedy_head_ties_go_to_the_smallest_token(gpu):
    mmf = _mmf()
    k, vocab = 256, 1000
    w = synth.rng(840).standard_normal((vocab, k), dtype=np.float32) * np.float32(0.02)
    x = synth.activations((3, k), 841)
    x[1] = 0.0  # a zero row: every sum is 0
    w_same = np.repeat(w[:1], vocab, axis=0)  # identical rows: every sum equal
    for wt, want in ((w, None), (w_same, 0)):
        t, mu = oracle.ternarize(wt)
        ref = oracle.greedy_head(x, t, mu)["tokens"]
        got = host(mmf.greedy_head(dev(x, gpu), mmf.ternary_pack(dev(wt, gpu))))
        assert_equal(got, ref, "tokens")
        assert got[1] == 0
        if want is not None:
            assert np.all(got == want)


def test_generate_loop_stage_by_stage(gpu):
    """The token-to-token loop of a two-block model: embed -> decode steps -> greedy head. At
    every step the embedding is checked bit for bit and the head's tokens are checked bit for bit
    against the oracle fed with the GPU's last block output; the tokens feed the next step."""
    import torch
    mmf = _mmf()
    d, inner, vocab, b, L = 256, 512, 1000, 3, 2
    table = synth.activations((vocab, d), 850, "bf16")
    pairs = [make_pair(d, inner, 851 + l, gpu) for l in range(L)]
    w_head = synth.rng(853).standard_normal((vocab, d), dtype=np.float32) * np.float32(0.02)
    t_head, mu_head = oracle.ternarize(w_head)
    head = mmf.ternary_pack(dev(w_head, gpu))
    hs = [dev(synth.activations((b, d), 854 + l), gpu) for l in range(L)]
    td = bf16_tensor(table, gpu)
    ids = dev(np.array([1, 500, 999], dtype=np.int32), gpu)
    for step in range(4):
        x = mmf.embed(ids, td)
        assert_equal(host(x), oracle.embed(host(ids), table), "embed step %d" % step)
        y = x
        for l in range(L):
            y = mmf.layer_decode_step(pairs[l][1], y, hs[l])
        nxt = mmf.greedy_head(y, head)
        ref = oracle.greedy_head(host(y), t_head, mu_head)["tokens"]
        assert_equal(host(nxt), ref, "tokens step %d" % step)
        ids = nxt


LAYER_BWD_CASES = [
    # d, inner, b, t, act, gains, mode
    (256, 512, 2, 33, "f32", None, "recurrent"),
    (256, 512, 2, 70, "bf16", "distinct", "chunk"),
    (128, 352, 1, 300, "bf16", "shared", "auto"),
]


@pytest.mark.parametrize("d,inner,b,t,act,gains,mode", LAYER_BWD_CASES)
def test_layer_bwd_parity(gpu, d, inner, b, t, act, gains, mode):
    """Every derivative of the block (straight-through quantisers) against the oracle's chain,
    evaluated at the GPU forward's own stage values (a probed forward call runs the kernels the
    derivative's recompute runs), so that both sides' quantisers see the same inputs. The
    products run in bf16: the bf16 bar applies (rtol 2e-2)."""
    mmf = _mmf()
    L, P = make_pair(d, inner, 860 + t, gpu, gains)
    x = synth.activations((b, t, d), 861, act)
    dout = synth.activations((b, t, d), 862, act)
    h0 = synth.activations((b, d), 863)
    dhl = synth.activations((b, d), 864)
    xd = bf16_tensor(x, gpu) if act == "bf16" else dev(x, gpu)
    m = b * t
    probe = mmf.LayerProbe(m, d, inner, gpu, shared_ifg=gains != "distinct")
    mmf.layer_fwd(P, xd, dev(h0, gpu), mode=mode, probe=probe)
    pr = probe.host()
    i_hat = oracle.dequant(pr["acc_ifg"].reshape(m, 3, d)[:, 0], pr["scale_x"][0], L.i.mu)
    ab = oracle.dequant(pr["acc_gate"], pr["scale_x1"], L.gate.mu)
    stages = dict(i_hat=i_hat, f=pr["f"], g=pr["g"], h=pr["h"], u=pr["u"], x1=pr["x1"], ab=ab, z=pr["z"])
    ref = oracle.layer_backward(L, x, dout, h0, dhl, stages=stages)
    dod = bf16_tensor(dout, gpu) if act == "bf16" else dev(dout, gpu)
    got = mmf.layer_bwd(P, xd, dod, dev(h0, gpu), dev(dhl, gpu), mode, want_gains=True)
    tol = 2e-2
    assert_close(host(got["dx"]), ref["dx"], tol, "dx")
    assert_close(host(got["dh0"]), ref["dh0"], tol, "dh0")
    assert_close(host(got["dg_norm_w"]), ref["dg_norm_w"], tol, "dg_norm_w")
    for k in ("i", "f", "g", "o", "gate", "down"):
        assert_close(host(got["dw"][k]), ref["dw"][k], tol, "dw " + k)
        assert_close(host(got["dgain"][k]), ref["dgain"][k], tol, "dgain " + k)
    path = mmf.last_path()
    assert "gemm_bf16<dw>" in path and ("scan_bwd_recurrent" if mode == "recurrent" else "scan_bwd") in path


def test_layer_bwd_empty_sequence(gpu):
    import torch
    mmf = _mmf()
    _, P = make_pair(64, 96, 870, gpu)
    dhl = dev(synth.activations((2, 64), 871), gpu)
    e = torch.empty((2, 0, 64), device=gpu)
    got = mmf.layer_bwd(P, e, e, None, dhl, want_gains=True)
    assert torch.equal(got["dh0"], dhl)
    assert not host(got["dw"]["gate"]).any() and not host(got["dg_norm_w"]).any()


SCAN_BWD_CASES = [
    # b, t, d, mode, with_h0, with_last
    (1, 1, 64, "recurrent", True, True),
    (2, 7, 48, "recurrent", False, True),
    (3, 300, 96, "recurrent", True, False),
    (4, 63, 256, "auto", True, True),        # auto below 64 steps: recurrent
    (2, 300, 96, "chunk", True, True),       # few groups: 16-wave workgroups
    (1, 4099, 128, "chunk", True, True),     # T >= 4096
    (8, 700, 1024, "chunk", True, True),     # ragged last chunk
    (16, 300, 520, "auto", False, True),     # partial channel group
    (2, 4100, 4096, "chunk", True, False),   # streaming accesses
    (16, 260, 2048, "chunk", True, True),    # many groups: 4-wave workgroups, ragged last chunk
]


def _scan_bwd_inputs(b, t, d, seed, with_h0, with_last):
    """f and the forward's h (the oracle's, rounded to binary32), an upstream dh, and optional
    h0 and dh_last, all seeded."""
    x, f = synth.scan_inputs(b, t, d, seed)
    h0 = synth.activations((b, d), seed + 1) if with_h0 else None
    h = oracle.hgrn_scan(x, f, h0).astype(np.float32)
    dh = synth.activations((b, t, d), seed + 2)
    gl = synth.activations((b, d), seed + 3) if with_last else None
    return f, h, dh, h0, gl


@pytest.mark.parametrize("b,t,d,mode,with_h0,with_last", SCAN_BWD_CASES)
def test_scan_bwd_parity(gpu, b, t, d, mode, with_h0, with_last):
    mmf = _mmf()
    f, h, dh, h0, gl = _scan_bwd_inputs(b, t, d, 700 + t + d, with_h0, with_last)
    dx, df, dh0 = mmf.hgrn_scan_bwd(dev(f, gpu), dev(h, gpu), dev(dh, gpu), dev(h0, gpu) if with_h0 else None,
                                    dev(gl, gpu) if with_last else None, mode, want_dh0=True)
    rdx, rdf, rdh0 = oracle.hgrn_scan_bwd(f, h, dh, h0, gl)
    rtol = 1e-3 if (mode != "recurrent" and t >= 4096) else 1e-4
    assert_close(host(dx), rdx, rtol, "dx")
    assert_close(host(df), rdf, rtol, "df")
    assert_close(host(dh0), rdh0, rtol, "dh0")
    path = mmf.last_path()
    if mode == "recurrent" or (mode == "auto" and t < 64):
        assert "scan_bwd_recurrent" in path, path
    else:
        assert "scan_bwd_tiled" in path, path


def test_scan_bwd_in_place_empty_and_limits(gpu):
    import torch
    mmf = _mmf()
    f, h, dh, h0, gl = _scan_bwd_inputs(4, 390, 2048, 704, True, True)
    rdx, rdf, rdh0 = oracle.hgrn_scan_bwd(f, h, dh, h0, gl)
    for mode in ("recurrent", "chunk"):
        dhd = dev(dh, gpu)
        dx, df, dh0 = mmf.hgrn_scan_bwd(dev(f, gpu), dev(h, gpu), dhd, dev(h0, gpu), dev(gl, gpu), mode, dx=dhd,
                                        want_dh0=True)
        assert dx.data_ptr() == dhd.data_ptr()
        assert_close(host(dx), rdx, 1e-4, "in-place dx " + mode)
        assert_close(host(df), rdf, 1e-4, "in-place df " + mode)
        assert_close(host(dh0), rdh0, 1e-4, "in-place dh0 " + mode)
    # no steps: h_last is h0, so dh0 = dh_last
    e = torch.empty((2, 0, 64), device=gpu)
    gl2 = dev(synth.activations((2, 64), 706), gpu)
    _, _, dh0 = mmf.hgrn_scan_bwd(e, e, e, None, gl2, want_dh0=True)
    assert torch.equal(dh0, gl2)
    # f = 0: nothing reaches back, dx = dh (+ dh_last on the last step), dh0 = 0
    zero = np.zeros((2, 257, 64), dtype=np.float32)
    dh3 = synth.activations((2, 257, 64), 707)
    h3 = synth.activations((2, 257, 64), 708)
    gl3 = synth.activations((2, 64), 709)
    for mode in ("recurrent", "chunk"):
        dx, _, dh0 = mmf.hgrn_scan_bwd(dev(zero, gpu), dev(h3, gpu), dev(dh3, gpu), None, dev(gl3, gpu), mode,
                                       want_dh0=True)
        want = dh3.copy()
        want[:, -1] += gl3
        assert np.array_equal(host(dx), want), mode
        assert not host(dh0).any(), mode


def test_scan_bwd_c5_full_size_sampled(gpu):
    """The backward at the long-sequence stress shape (B=16, T=32768, d=2048, f = sigmoid(N(2,1))),
    chunked: h from the forward kernel, dh ~ N(0, 1); the oracle runs whole sequences for 64
    sampled channels (4 per sequence) from the same f, h and dh."""
    import torch
    mmf = _mmf()
    b, t, d = 16, 32768, 2048
    fd = torch.empty((b, t, d), device=gpu)
    hd = torch.empty((b, t, d), device=gpu)
    dhd = torch.empty((b, t, d), device=gpu)
    pick = np.stack([synth.rng(7500 + i).choice(d, size=4, replace=False) for i in range(b)])
    fs, dhs = [], []
    for i in range(b):
        x, f = synth.scan_inputs(1, t, d, 7 * 1000 + i)
        hd[i].copy_(torch.from_numpy(x[0]))  # x for now; the forward overwrites it with h
        fd[i].copy_(torch.from_numpy(f[0]))
        fs.append(f[0][:, pick[i]].copy())
        del x, f
        g = synth.activations((t, d), 7 * 1000 + 500 + i)
        dhd[i].copy_(torch.from_numpy(g))
        dhs.append(g[:, pick[i]].copy())
        del g
    mmf.hgrn_scan_fwd(hd, fd, None, "chunk", out=hd)
    dx, df, dh0 = mmf.hgrn_scan_bwd(fd, hd, dhd, None, None, "chunk", want_dh0=True)
    assert "scan_bwd_tiled" in mmf.last_path()
    idx = torch.from_numpy(pick).to(gpu)
    sel = idx[:, None, :].expand(b, t, 4)
    hs = torch.gather(hd, 2, sel).cpu().numpy()
    got_dx = torch.gather(dx, 2, sel).cpu().numpy()
    got_df = torch.gather(df, 2, sel).cpu().numpy()
    got_dh0 = torch.gather(dh0, 1, idx).cpu().numpy()
    rdx, rdf, rdh0 = oracle.hgrn_scan_bwd(np.stack(fs), hs, np.stack(dhs))
    assert_close(got_dx, rdx, 1e-3, "dx (sampled channels)")
    assert_close(got_df, rdf, 1e-3, "df (sampled channels)")
    assert_close(got_dh0, rdh0, 1e-3, "dh0 (sampled channels)")


LAYER_CASES = [
    # d, inner, b, t, act, gains, mode
    (64, 96, 1, 1, "f32", None, "recurrent"),
    (256, 512, 2, 33, "f32", None, "recurrent"),
    (256, 512, 2, 33, "bf16", "shared", "chunk"),
    (128, 352, 3, 70, "f32", "distinct", "recurrent"),
    (128, 352, 1, 300, "bf16", "distinct", "chunk"),
]


@pytest.mark.parametrize("d,inner,b,t,act,gains,mode", LAYER_CASES)
def test_layer_stages(gpu, d, inner, b, t, act, gains, mode):
    import torch
    mmf = _mmf()
    L, P = make_pair(d, inner, 500 + d + t, gpu, gains)
    x = synth.activations((b, t, d), 501, act)
    h0 = synth.activations((b, d), 502)
    probe = mmf.LayerProbe(b * t, d, inner, gpu, shared_ifg=(gains != "distinct"))
    xd = bf16_tensor(x, gpu) if act == "bf16" else dev(x, gpu)
    out, h_last = mmf.layer_fwd(P, xd, dev(h0, gpu), mode=mode, probe=probe)
    torch.cuda.synchronize()
    pr = probe.host()
    check_layer_stages(L, x, h0, pr, host(out), act, shared=(gains != "distinct"))
    assert_close(host(h_last), pr["h"].reshape(b, t, d)[:, -1], 0, "h_last")


def test_stack_of_blocks_stage_fed(gpu):
    """A stack of three blocks of the 370M width, bf16, each block's output feeding the next (the
    stack the benchmark runs): every block is checked stage by stage against the oracle fed with
    the GPU's input to that block, and its output is the next block's input bit for bit."""
    import torch
    mmf = _mmf()
    d, inner, b, t = 1024, 2816, 2, 96
    pairs = [make_pair(d, inner, synth.layer_seed(2, l), gpu) for l in range(3)]
    cur = bf16_tensor(synth.activations((b, t, d), 21, "bf16"), gpu)
    for l, (L, P) in enumerate(pairs):
        probe = mmf.LayerProbe(b * t, d, inner, gpu)
        x_in = host(cur)
        out, _ = mmf.layer_fwd(P, cur, None, want_h_last=True, mode="chunk", probe=probe)
        torch.cuda.synchronize()
        check_layer_stages(L, x_in, None, probe.host(), host(out), "bf16")
        cur = out
    assert cur.dtype == torch.bfloat16


def test_layer_c1_end_to_end(gpu):
    """370M-width layer, fp32, batch 1, T=128, recurrent scan: stage-fed and free-running against the oracle."""
    import torch
    mmf = _mmf()
    d, inner = 1024, 2816
    L, P = make_pair(d, inner, synth.layer_seed(1, 0), gpu)
    x = synth.activations((1, 128, d), 1)
    probe = mmf.LayerProbe(128, d, inner, gpu)
    out, h_last = mmf.layer_fwd(P, dev(x, gpu), None, mode="recurrent", probe=probe)
    torch.cuda.synchronize()
    pr = probe.host()
    outg = host(out).reshape(128, d)
    check_layer_stages(L, x, None, pr, outg, "f32")
    # free-running oracle: the input codes are identical; later quantisers see inputs that differ
    # by rounding only, so a code may flip where y*s lies within rounding of a half-integer
    check_free_running(pr, oracle.layer_forward(L, x), outg, "f32")


DECODE_CASES = [
    # b, act, gains, d, inner, expected kernel family
    (1, "bf16", "shared", 256, 512, "tgemv"),
    (5, "f32", None, 272, 1040, "tgemv"),
    (16, "bf16", "shared", 256, 512, "tgemv"),
    (16, "bf16", "distinct", 256, 512, "tgemv"),
    (17, "f32", "shared", 256, 512, "tgemv"),
    (64, "bf16", "shared", 256, 512, "tgemv"),
    (65, "bf16", "shared", 256, 512, "tgemm"),
    (3, "bf16", "shared", 256, 4160, "tgemv"),      # wide down_proj input rows
    (1, "bf16", None, 2048, 5632, "tgemv"),         # the 1.3B decode shape at its three batches
    (16, "bf16", None, 2048, 5632, "tgemv"),
    (64, "bf16", None, 2048, 5632, "tgemv"),
    (8, "bf16", None, 2560, 6912, "tgemv"),         # the 2.7B decode shape
]


@pytest.mark.parametrize("b,act,gains,d,inner,family", DECODE_CASES)
def test_decode_step_stages(gpu, b, act, gains, d, inner, family):
    import torch
    mmf = _mmf()
    L, P = make_pair(d, inner, 600 + b, gpu, gains)
    x = synth.activations((b, d), 601, act)
    h0 = synth.activations((b, d), 602)
    hd = dev(h0, gpu)
    shared = gains != "distinct"
    probe = mmf.LayerProbe(b, d, inner, gpu, shared_ifg=shared)
    xd = bf16_tensor(x, gpu) if act == "bf16" else dev(x, gpu)
    h_plain = hd.clone()
    out_plain = mmf.layer_decode_step(P, xd, h_plain)
    path_plain = mmf.last_path()
    out = mmf.layer_decode_step(P, xd, hd, probe=probe)
    torch.cuda.synchronize()
    assert family in mmf.last_path(), mmf.last_path()
    # a probe changes neither the kernels the default path launches nor their bits
    assert mmf.last_path() == path_plain, (mmf.last_path(), path_plain)
    assert torch.equal(out, out_plain) and torch.equal(hd, h_plain)
    pr = probe.host()
    check_layer_stages(L, x[:, None, :], h0, pr, host(out), act, shared=shared)
    assert np.array_equal(host(hd), pr["h"])


@pytest.mark.parametrize("b,act,gains,d,inner", [(1, "bf16", None, 2048, 5632), (16, "bf16", None, 2048, 5632),
                                                  (5, "f32", "shared", 272, 1040), (1, "f32", ("o", "g_norm"), 272, 1040)])
def test_decode_step_stages_separate(gpu, b, act, gains, d, inner):
    """The separate-kernel decode step (mmf_set_decode_kernel 1) stage by stage."""
    import torch
    mmf = _mmf()
    L, P = make_pair(d, inner, 650 + b, gpu, gains)
    x = synth.activations((b, d), 651, act)
    h0 = synth.activations((b, d), 652)
    hd = dev(h0, gpu)
    probe = mmf.LayerProbe(b, d, inner, gpu)
    xd = bf16_tensor(x, gpu) if act == "bf16" else dev(x, gpu)
    try:
        mmf.set_decode_kernel("separate")
        out = mmf.layer_decode_step(P, xd, hd, probe=probe)
        torch.cuda.synchronize()
        assert "tgemv_row" not in mmf.last_path() and "norm_quant_row" in mmf.last_path(), mmf.last_path()
    finally:
        mmf.set_decode_kernel("auto")
    pr = probe.host()
    check_layer_stages(L, x[:, None, :], h0, pr, host(out), act)
    assert np.array_equal(host(hd), pr["h"])


def test_decode_512_steps_then_stages(gpu):
    """The decode sequence length of the 1.3B decode workload: 512 steps of one layer at batch 16
    from a carried state h ~ N(0, 1), then the 513th step checked stage by stage."""
    import torch
    mmf = _mmf()
    d, inner, b = 2048, 5632, 16
    L, P = make_pair(d, inner, 3000, gpu)
    h = dev(synth.activations((b, d), 3001), gpu)
    xs = synth.activations((513, b, d), 3002, "bf16")
    xd = bf16_tensor(xs, gpu)
    ws = torch.empty(mmf.layer_workspace_size(P, b, 1), dtype=torch.uint8, device=gpu)
    out = torch.empty((b, d), dtype=torch.bfloat16, device=gpu)
    for s_ in range(512):
        mmf.layer_decode_step(P, xd[s_], h, out=out, ws=ws)
    h_before = host(h)
    assert np.all(np.isfinite(h_before))
    probe = mmf.LayerProbe(b, d, inner, gpu)
    out = mmf.layer_decode_step(P, xd[512], h, probe=probe, ws=ws)
    torch.cuda.synchronize()
    check_layer_stages(L, xs[512][:, None, :], h_before, probe.host(), host(out), "bf16")


FULL_SIZE_PREFILL = [
    # shape, batch, tokens, config seed: one layer of each prefill workload at full size, bf16,
    # in the launch configuration the benchmark uses (scan mode auto)
    ("370M", 8, 2048, 2),
    ("1.3B", 16, 2048, 3),
    ("2.7B", 4, 4096, 4),
]


@pytest.mark.parametrize("shape,b,t,seed", FULL_SIZE_PREFILL)
def test_layer_full_size_sampled(gpu, shape, b, t, seed):
    """One layer at full size in the benchmark's launch configuration (no probe: the typed fast
    epilogues), then again with a probe (the generic epilogues the stage checks read): both give
    the same bits. Every stage of one sampled token per 128-row tile of the contractions (and
    the first and last token) is checked against the oracle fed with the GPU's stage inputs, and
    the scan over whole sequences for 6 sampled channels."""
    import torch
    mmf = _mmf()
    d, inner, _ = synth.SHAPES[shape]
    L, P = make_pair(d, inner, synth.layer_seed(seed, 0), gpu)
    xs = synth.activations((b, t, d), seed * 10 + 1, "bf16")
    xd = bf16_tensor(xs, gpu)
    out_plain, hl_plain = mmf.layer_fwd(P, xd, None, want_h_last=True, mode="auto")
    torch.cuda.synchronize()
    path_plain = mmf.last_path()
    probe = mmf.LayerProbe(b * t, d, inner, gpu)
    out, hl = mmf.layer_fwd(P, xd, None, want_h_last=True, mode="auto", probe=probe)
    torch.cuda.synchronize()
    path = mmf.last_path()
    assert path == path_plain, (path, path_plain)
    assert "tgemm_dma" in path and "scan_tiled" in path, path
    assert torch.equal(out_plain, out) and torch.equal(hl_plain, hl)
    del out_plain, hl_plain
    m = b * t
    r = synth.rng(seed * 10 + 7)
    rows = {int(r.integers(s0, min(s0 + 128, m))) for s0 in range(0, m, 128)} | {0, m - 1}
    chans = [(int(r.integers(b)), int(r.integers(d))) for _ in range(6)]
    check_layer_sampled(L, xs, None, probe, out, "bf16", b, t, rows, chans,
                        scan_rtol=1e-3 if t >= 4096 else 1e-4)


def test_decode_steps_equal_prefill(gpu):
    """T decode steps with the carried state reproduce a recurrent-mode prefill bit for bit (fp32)."""
    import torch
    mmf = _mmf()
    d, inner, b, t = 128, 256, 3, 12
    _, P = make_pair(d, inner, 700, gpu, "distinct")
    x = dev(synth.activations((b, t, d), 701), gpu)
    h0 = dev(synth.activations((b, d), 702), gpu)
    out, h_last = mmf.layer_fwd(P, x, h0, mode="recurrent")
    h = h0.clone()
    outs = [mmf.layer_decode_step(P, x[:, s].contiguous(), h) for s in range(t)]
    torch.cuda.synchronize()
    assert torch.equal(torch.stack(outs, 1), out)
    assert torch.equal(h, h_last)


def test_decode_resume_is_bit_identical(gpu):
    import torch
    mmf = _mmf()
    d, inner, b = 128, 256, 2
    _, P = make_pair(d, inner, 710, gpu)
    xs = dev(synth.activations((16, b, d), 711, "bf16"), gpu).to(torch.bfloat16)
    h = dev(synth.activations((b, d), 712), gpu)
    h_a = h.clone()
    full = [mmf.layer_decode_step(P, xs[s], h_a) for s in range(16)]
    h_b = h.clone()
    part = [mmf.layer_decode_step(P, xs[s], h_b) for s in range(8)]
    saved = h_b.cpu()
    h_c = saved.to(gpu)
    part += [mmf.layer_decode_step(P, xs[s], h_c) for s in range(8, 16)]
    torch.cuda.synchronize()
    assert torch.equal(torch.stack(full), torch.stack(part))
    assert torch.equal(h_a, h_c)


def test_layer_deterministic(gpu):
    import torch
    mmf = _mmf()
    d, inner, b, t = 256, 512, 2, 200
    _, P = make_pair(d, inner, 720, gpu)
    x = bf16_tensor(synth.activations((b, t, d), 721, "bf16"), gpu)
    runs = [mmf.layer_fwd(P, x, None, mode="chunk") for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])


@pytest.mark.parametrize("d,inner,b,t,act,gains", [
    (256, 512, 2, 100, "bf16", None),        # ragged tiles
    (256, 512, 2, 128, "bf16", "shared"),    # whole tiles
    (128, 352, 3, 70, "f32", "distinct"),    # split activations, fp32
    (512, 1024, 1, 256, "f32", None),
])
def test_layer_probe_does_not_change_results(gpu, d, inner, b, t, act, gains):
    """Without a probe the contractions take the typed fast epilogue; with one, the
    generic epilogue that the stage checks cover. Both must give the same bits."""
    import torch
    mmf = _mmf()
    _, P = make_pair(d, inner, 730 + t, gpu, gains)
    xs = synth.activations((b, t, d), 731 + t, act)
    x = bf16_tensor(xs, gpu) if act == "bf16" else dev(xs, gpu)
    h0 = dev(synth.activations((b, d), 732), gpu)
    out_a, hl_a = mmf.layer_fwd(P, x, h0, want_h_last=True, mode="chunk")
    probe = mmf.LayerProbe(b * t, d, inner, gpu, shared_ifg=gains != "distinct")
    out_b, hl_b = mmf.layer_fwd(P, x, h0, want_h_last=True, mode="chunk", probe=probe)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    assert torch.equal(hl_a, hl_b)


@pytest.mark.parametrize("m,k,n,dt", [(300, 256, 200, "bf16"), (256, 512, 256, "f32"), (130, 2048, 4096, "bf16")])
def test_bitlinear_probe_does_not_change_results(gpu, m, k, n, dt):
    import torch
    mmf = _mmf()
    w = synth.rng(741 + m).standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    pl = mmf.ternary_pack(dev(w, gpu))
    xs = synth.activations((m, k), 742 + m, dt)
    x = bf16_tensor(xs, gpu) if dt == "bf16" else dev(xs, gpu)
    y_a = mmf.bitlinear_fwd(x, pl)
    acc = torch.empty((m, n), dtype=torch.int32, device=gpu)
    y_b = mmf.bitlinear_fwd(x, pl, acc_out=acc)
    torch.cuda.synchronize()
    assert torch.equal(y_a, y_b)


def test_layer_empty_sequence(gpu):
    import torch
    mmf = _mmf()
    _, P = make_pair(64, 96, 730, gpu)
    h0 = dev(synth.activations((2, 64), 731), gpu)
    out, h_last = mmf.layer_fwd(P, torch.empty((2, 0, 64), device=gpu), h0)
    torch.cuda.synchronize()
    assert out.shape == (2, 0, 64) and torch.equal(h_last, h0)


def _graph_replays(P, x, h0, mark, gpu):
    """Captures one decode step and replays it with eager work between replays; every replay
    must give the eager result."""
    import torch
    mmf = _mmf()
    b, d = x.shape
    ws = torch.empty(mmf.layer_workspace_size(P, b, 1), dtype=torch.uint8, device=gpu)
    out = torch.empty((b, d), dtype=x.dtype, device=gpu)
    h = h0.clone()
    mmf.layer_decode_step(P, x, h, out=out, ws=ws)  # eager
    assert mark in mmf.last_path()
    ref_out, ref_h = out.clone(), h.clone()
    g = torch.cuda.CUDAGraph()
    h.copy_(h0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        mmf.layer_decode_step(P, x, h, out=out, ws=ws)
    for _ in range(4):
        h.copy_(h0)
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(h, ref_h)
        mmf.layer_fwd(P, x[:, None, :].contiguous(), None)  # unrelated eager work between replays


@pytest.mark.parametrize("b", [16, 64])
def test_decode_separate_graph_replays(gpu, b):
    """The default decode step (the path the benchmark replays) at the 1.3B shape: captured once,
    replayed several times with eager work between, every replay equals the eager result."""
    _, P = make_pair(2048, 5632, 940 + b, gpu)
    x = bf16_tensor(synth.activations((b, 2048), 941, "bf16"), gpu)
    h0 = dev(synth.activations((b, 2048), 942), gpu)
    _graph_replays(P, x, h0, "tgemv<", gpu)


def test_generate_step_graph_replays(gpu):
    """One token-to-token step (embed, two blocks, greedy head) captured and replayed from the
    same ids and states: every replay gives the eager tokens and states."""
    import torch
    mmf = _mmf()
    d, inner, vocab, b, L = 256, 512, 1000, 4, 2
    table = bf16_tensor(synth.activations((vocab, d), 950, "bf16"), gpu)
    Ps = [make_pair(d, inner, 951 + l, gpu)[1] for l in range(L)]
    head = mmf.ternary_pack(dev(synth.rng(953).standard_normal((vocab, d), dtype=np.float32) * np.float32(0.02), gpu))
    ids0 = dev(np.array([3, 77, 500, 999], dtype=np.int32), gpu)
    h0 = [dev(synth.activations((b, d), 954 + l), gpu) for l in range(L)]
    ids, hs = ids0.clone(), [h.clone() for h in h0]
    x = torch.empty((b, d), dtype=torch.bfloat16, device=gpu)
    outs = [torch.empty_like(x) for _ in range(2)]
    ws = torch.empty(mmf.layer_workspace_size(Ps[0], b, 1), dtype=torch.uint8, device=gpu)

    def step():
        mmf.embed(ids, table, out=x)
        y = x
        for l in range(L):
            y = mmf.layer_decode_step(Ps[l], y, hs[l], out=outs[l % 2], ws=ws)
        mmf.greedy_head(y, head, tokens=ids)

    step()
    torch.cuda.synchronize()
    ref_ids, ref_hs = ids.clone(), [h.clone() for h in hs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(4):
        ids.copy_(ids0)
        for h, h_init in zip(hs, h0):
            h.copy_(h_init)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ids, ref_ids)
        assert all(torch.equal(h, r) for h, r in zip(hs, ref_hs))
        mmf.bitlinear_fwd(x, head)  # unrelated eager work between replays


ROW_CASES = [
    # b, d, inner, act, gains: without gains on i/f/g, gate_proj and down_proj the contractions
    # quantise their own input rows where cheap; o_proj forms the gated g_norm itself unless it
    # has a gain
    (1, 256, 512, "bf16", None),
    (1, 272, 1040, "f32", ("g_norm",)),  # slices past the row end; g_norm's gain
    (1, 2048, 5632, "bf16", None),       # the 1.3B decode shape
    (1, 2560, 6912, "f32", None),        # the 2.7B width, two slices per wave in down_proj
    (2, 2048, 5632, "bf16", ("g_norm",)),  # a wave per row
    (5, 272, 1040, "f32", ("o",)),       # o_proj's gain: the g_norm quantiser runs
    (16, 2048, 5632, "bf16", None),      # the 1.3B decode batch: down_proj's rows too wide
    (16, 1024, 2816, "f32", ("g_norm", "o")),
    (8, 2560, 6912, "bf16", None),       # rows wider than 2048: the separate quantisers
    (1, 16, 32, "bf16", ("g_norm",)),    # one packed word per row
    (1, 2048, 5632, "bf16", "shared"),   # gains: each one-row contraction applies its own
    (1, 272, 1040, "f32", ("gate",)),
    (1, 272, 1040, "f32", ("o", "g_norm")),  # o_proj's gain after the gated g_norm
    (1, 4608, 256, "f32", ("o", "g_norm")),  # ... with two slices per wave in o_proj
    (4, 256, 512, "bf16", ("down",)),    # several rows with a gain
    (16, 2048, 5632, "bf16", "shared"),  # more than 12 rows with gains: the separate quantisers
    (12, 2048, 2048, "f32", ("i", "gate", "down")),
    (3, 16, 48, "f32", None),
    (16, 48, 16, "bf16", None),          # 16 rows of three words; down_proj over one word
    (9, 1024, 2816, "bf16", None),       # i/f/g's rows in two workgroups per channel block: 8 + 1
    (13, 272, 1040, "f32", None),        # ... 8 + 5, in i/f/g, gate_proj and down_proj, rows not whole chunks
]


@pytest.mark.parametrize("b,d,inner,act,gains", ROW_CASES)
def test_decode_row_path_matches_separate(gpu, b, d, inner, act, gains):
    """The default decode step lets i/f/g, gate_proj and down_proj quantise their own input rows
    where that is cheaper than a quantiser launch (one row; up to 16 rows of at most 2048), and
    o_proj form and quantise the gated g_norm of one row; over a chain of steps it must give the
    separate kernels' outputs and states bit for bit."""
    import torch
    mmf = _mmf()
    _, P = make_pair(d, inner, 970 + d, gpu, gains)
    xs = [synth.activations((b, d), 971 + s_, act) for s_ in range(4)]
    h0 = synth.activations((b, d), 975)
    res = {}
    for mode in ("auto", "separate"):
        mmf.set_decode_kernel(mode)
        try:
            h = dev(h0, gpu)
            outs = []
            for xv in xs:
                xd = bf16_tensor(xv, gpu) if act == "bf16" else dev(xv, gpu)
                outs.append(host(mmf.layer_decode_step(P, xd, h)))
                if mode == "auto":
                    steps = mmf.last_path().split(";")
                    fused = [k for k in steps if k.startswith("tgemv_row<")]
                    widest = 8192 if b == 1 else 2048  # widest input row a contraction quantises itself
                    # a stage is fused where its row fits, with or without its gain; o_proj forms the
                    # gated g_norm (then applies its own gain) at one row
                    def gain(name):
                        return gains == "shared" or (isinstance(gains, tuple) and name in gains)
                    # more than 12 rows with a gain keep the separate quantiser
                    stages = (("gates_step", d, gain("i")), ("resid,gnorm", d if b == 1 else 1 << 30, False),
                              ("glu", d, gain("gate")), ("resid", inner, gain("down")))
                    want = [e for e, k, g in stages if k <= widest and not (g and b > 12)]
                    assert fused == ["tgemv_row<%s>" % e for e in want], steps
                    quant = [k for k in steps if "norm_quant" in k]
                    assert len(quant) == 4 - len(want), steps
            torch.cuda.synchronize()
            res[mode] = (outs, host(h))
        finally:
            mmf.set_decode_kernel("auto")
    for a_, b_ in zip(res["auto"][0], res["separate"][0]):
        assert_equal(a_, b_, "out")
    assert_equal(res["auto"][1], res["separate"][1], "h")


@pytest.mark.parametrize("b,act,gains", [(1, "f32", None), (1, "bf16", ("g_norm",)), (16, "f32", None),
                                          (16, "bf16", None), (64, "bf16", None), (64, "f32", None),
                                          (1, "f32", "shared"), (1, "bf16", "shared"), (12, "bf16", "shared")])
def test_decode_default_path_end_to_end(gpu, b, act, gains):
    """The default decode step at the 1.3B shape (at b <= 16 the contractions that quantise their
    own rows) against the unmodified oracle run free: the state within fp32 rounding (it depends
    only on the first quantiser, whose input is the same on both sides); the output elementwise
    within the activation type's tolerance on every row without a code flip, normwise on all.
    The probe that names the flipped rows does not change the kernels or their bits: the same
    step without it gives the same output and state."""
    import torch
    mmf = _mmf()
    d, inner = 2048, 5632
    L, P = make_pair(d, inner, 1900 + b, gpu, gains)
    x = synth.activations((b, d), 1901, act)
    h0 = synth.activations((b, d), 1902)
    xd = bf16_tensor(x, gpu) if act == "bf16" else dev(x, gpu)
    h = dev(h0, gpu)
    out = mmf.layer_decode_step(P, xd, h)
    path_plain = mmf.last_path()
    hp = dev(h0, gpu)
    probe = mmf.LayerProbe(b, d, inner, gpu)
    outp = mmf.layer_decode_step(P, xd, hp, probe=probe)
    torch.cuda.synchronize()
    assert mmf.last_path() == path_plain, (mmf.last_path(), path_plain)
    assert ("tgemv_row<" in path_plain) == (b <= 16), path_plain
    assert torch.equal(out, outp) and torch.equal(h, hp)
    pr = probe.host()
    check_layer_stages(L, x[:, None, :], h0, pr, host(out), act)
    ref = oracle.layer_decode_step(L, x, h0)
    assert_close(host(h), ref["h"], 1e-4, "h")
    check_free_running(pr, ref["stages"], host(out), act)


def test_decode_row_path_needs_few_rows_and_one_ifg_gain(gpu):
    mmf = _mmf()
    _, P = make_pair(256, 512, 980, gpu, "distinct")  # i/f/g gains differ: three quantisations of x
    x = bf16_tensor(synth.activations((1, 256), 981, "bf16"), gpu)
    mmf.layer_decode_step(P, x, dev(synth.activations((1, 256), 982), gpu))
    assert "tgemv_row" not in mmf.last_path()
    _, P2 = make_pair(256, 512, 983, gpu)
    x2 = bf16_tensor(synth.activations((17, 256), 984, "bf16"), gpu)  # more than one row block
    mmf.layer_decode_step(P2, x2, dev(synth.activations((17, 256), 985), gpu))
    assert "tgemv_row" not in mmf.last_path()


@pytest.mark.parametrize("b", [1, 16])
def test_decode_row_path_graph_replays(gpu, b):
    _, P = make_pair(2048, 5632, 990, gpu)
    x = bf16_tensor(synth.activations((b, 2048), 991, "bf16"), gpu)
    h0 = dev(synth.activations((b, 2048), 992), gpu)
    _graph_replays(P, x, h0, "tgemv_row<", gpu)


@pytest.mark.timeout(900)
def test_stack_1p3b_decode_step_24_layers_stage_fed(gpu):
    """One decode step of the whole 24-layer 1.3B stack at batch 16 on the default path (the
    graph the benchmark replays, here eager with a probe per layer): every layer is checked
    stage by stage against the oracle fed with the GPU's input to that layer and its carried
    state, and is checked free-running against the unmodified oracle step; its output is the
    next layer's input."""
    import torch
    mmf = _mmf()
    d, inner, L_, b = 2048, 5632, 24, 16
    cur_np = synth.activations((b, d), 3 * 10 + 2, "bf16")
    cur = bf16_tensor(cur_np, gpu)
    ws = None
    flips = 0
    for l in range(L_):
        L, P = make_pair(d, inner, synth.layer_seed(3, l), gpu)
        if ws is None:
            ws = torch.empty(mmf.layer_workspace_size(P, b, 1), dtype=torch.uint8, device=gpu)
        h0 = synth.activations((b, d), 3 * 100 + l)
        h = dev(h0, gpu)
        probe = mmf.LayerProbe(b, d, inner, gpu)
        x_in = host(cur)
        out = mmf.layer_decode_step(P, cur, h, probe=probe, ws=ws)
        torch.cuda.synchronize()
        assert "tgemv_row<" in mmf.last_path(), (l, mmf.last_path())
        pr = probe.host()
        check_layer_stages(L, x_in[:, None, :], h0, pr, host(out), "bf16")
        assert np.array_equal(host(h), pr["h"])
        flips += check_free_running(pr, oracle.layer_decode_step(L, x_in, h0)["stages"], host(out), "bf16",
                                    "out of layer %d" % l)
        cur = out
        del L, P
    # a flip needs a quantiser input within rounding of a half-integer decision point: a small
    # share of the rows, never most of them
    assert flips < L_ * b // 2, flips


@pytest.mark.timeout(900)
def test_stack_370m_prefill_24_layers_stage_fed(gpu):
    """The 24-layer 370M-width prefill stack (bf16, chunked scan, the kernels the benchmark's
    370M leg runs) at a reduced length: every block checked stage by stage against the oracle
    fed with the GPU's input to that block; each output is the next block's input."""
    import torch
    mmf = _mmf()
    d, inner, L_ = synth.SHAPES["370M"]
    b, t = 2, 160
    cur = bf16_tensor(synth.activations((b, t, d), 2 * 10 + 1, "bf16"), gpu)
    for l in range(L_):
        L, P = make_pair(d, inner, synth.layer_seed(2, l), gpu)
        probe = mmf.LayerProbe(b * t, d, inner, gpu)
        x_in = host(cur)
        out, _ = mmf.layer_fwd(P, cur, None, want_h_last=True, mode="chunk", probe=probe)
        torch.cuda.synchronize()
        assert "tgemm" in mmf.last_path(), mmf.last_path()
        check_layer_stages(L, x_in, None, probe.host(), host(out), "bf16")
        cur = out
        del L, P
    assert np.all(np.isfinite(host(cur)))


def test_mfma_ceiling_kernel(gpu):
    """The MFMA-only roof kernel: it reports the operations of its launch (4 workgroups of 4 waves
    per CU, each wave iters x 4 MFMAs of 2 * 32^3 operations), and every workgroup, doing the same
    arithmetic, writes the same sink word (written: two different fills are both overwritten)."""
    import torch
    mmf = _mmf()
    cus = torch.cuda.get_device_properties(gpu).multi_processor_count
    words = 4 * cus
    got = []
    for fill in (0, -1):
        sink = torch.full((words + 16,), fill, dtype=torch.int32, device=gpu)
        ops = mmf.mfma_ceiling(64, sink)
        torch.cuda.synchronize()
        assert ops == words * 4 * 64 * 4 * 2 * 32 ** 3
        w = sink.cpu().numpy()
        assert np.all(w[:words] == w[0]) and np.all(w[words:] == fill)
        got.append(int(w[0]))
    assert got[0] == got[1]
    sink = torch.zeros(words - 1, dtype=torch.int32, device=gpu)
    with pytest.raises(mmf.MMFError):
        mmf.mfma_ceiling(64, sink)


def test_hbm_ceiling_kernels_move_the_bytes(gpu):
    """The measured-roof kernels do what they time: the copy reproduces its source, the
    two-reads-one-write stream writes the XOR of its two sources, and the read stream's sink
    folds every word (ragged sizes exercise the tails)."""
    import torch
    mmf = _mmf()
    for nbytes in (16, 4096 + 48, 1 << 20):
        n = nbytes // 4
        g = torch.Generator(device=gpu)
        g.manual_seed(nbytes)
        src = torch.randint(-2 ** 31, 2 ** 31 - 1, (2 * n,), dtype=torch.int32, device=gpu, generator=g)
        dst = torch.empty(n, dtype=torch.int32, device=gpu)
        mmf.hbm_ceiling(src[:n], dst, "copy")
        torch.cuda.synchronize()
        assert torch.equal(dst, src[:n])
        mmf.hbm_ceiling(src, dst, "2r1w")
        torch.cuda.synchronize()
        assert torch.equal(dst, src[:n] ^ src[n:])
        sink = torch.zeros(8192, dtype=torch.int32, device=gpu)
        mmf.hbm_ceiling(src[:n], sink, "read")
        torch.cuda.synchronize()
        folded = 0
        for v in src[:n].cpu().numpy().tolist():
            folded ^= v
        total = 0
        for v in sink.cpu().numpy().tolist():
            total ^= v
        assert total == folded
