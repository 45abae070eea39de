"""Helpers shared by the GPU parity tests: device staging and the comparison rules.

Rules:
* integer and byte results (codes, packed words, int32 sums) must be equal;
* a quantiser's scale is compared bit for bit (same binary32 steps on both sides);
* real-valued results: |gpu - ref| <= rtol * (|ref| + RMS(ref)) elementwise.
"""
from __future__ import annotations

import numpy as np

import oracle
from ternary_weight_matmul_amd import synth


def assert_close(gpu, ref, rtol: float, what: str):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    if ref.size == 0:
        return
    assert np.all(np.isfinite(gpu)), what + ": non-finite values"
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(gpu - ref)
    bound = rtol * (np.abs(ref) + rms)
    bad = err > bound
    if bad.any():
        worst = float(np.max(err / np.maximum(bound, 1e-300)))
        raise AssertionError("%s: %d / %d elements beyond rtol %g (worst err/bound %.3g)" %
                             (what, int(bad.sum()), bad.size, rtol, worst))


def assert_equal(gpu, ref, what: str):
    gpu = np.asarray(gpu)
    ref = np.asarray(ref)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    if not np.array_equal(gpu, ref):
        idx = np.argwhere(gpu != ref)
        raise AssertionError("%s: %d / %d differ, first at %s: gpu %s ref %s" %
                             (what, len(idx), gpu.size, tuple(idx[0]), gpu[tuple(idx[0])], ref[tuple(idx[0])]))


def bf16_tensor(a, device):
    """float32 array whose values are bf16-exact -> torch bfloat16 tensor on device."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device).to(torch.bfloat16)


def dev(a, device, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return t if dtype is None else t.to(dtype)


def host(t):
    import torch
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def packed_words(pl) -> np.ndarray:
    return host(pl.packed).view(np.uint32)


def check_free_running(pr: dict, ref: dict, out_gpu: np.ndarray, act: str, what: str = "out"):
    """The GPU layer against the oracle run free (not fed with the GPU's stages). The first
    quantiser sees the same input on both sides, so its codes must be equal; a later quantiser's
    input differs by rounding only, so a code may flip by one where y*s lies within rounding of a
    half-integer (rare). Rows with no flipped code must match within the activation type's
    tolerance; a row with flips moves by a few quantisation steps at most (normwise bound)."""
    m = out_gpu.shape[0]
    assert_equal(pr["codes_x"][0], ref["q_i"].reshape(pr["codes_x"][0].shape), "codes_x (free-running)")
    flipped = np.zeros(m, bool)
    for key, rk in (("codes_u", "q_u"), ("codes_x1", "q_x1"), ("codes_z", "q_z")):
        r = ref[rk].reshape(pr[key].shape)
        diff = pr[key] != r
        assert np.all(np.abs(pr[key].astype(int) - r.astype(int))[diff] == 1), key
        assert diff.mean() < 1e-3, (key, diff.mean())
        flipped |= diff.any(axis=1)
    refo = ref["out"].reshape(m, -1)
    clean = ~flipped
    outg = np.asarray(out_gpu, np.float64)
    assert_close(outg[clean], refo[clean], 1e-4 if act == "f32" else 2e-2, what + " on rows without a code flip")
    rel = np.linalg.norm(outg - refo) / np.linalg.norm(refo)
    # bf16 output: its own rounding adds about 1.1e-3 normwise
    assert rel < (1e-3 if act == "f32" else 4e-3), (what, rel)
    return int(flipped.sum())


def make_pair(d, inner, seed, device, gains=None, eps=1e-8):
    """The same latent weights packed by the oracle (host) and by the GPU (mmf_ternary_pack)."""
    import ternary_weight_matmul_amd as mmf
    lat = synth.latent_weights(d, inner, seed)
    gn = None
    if gains == "shared":
        g = synth.norm_gains(d, inner, seed + 1)
        gn = {"i": g["i"], "f": g["i"], "g": g["i"], "o": g["o"], "gate": g["gate"], "down": g["down"],
              "g_norm": g["g_norm"]}
    elif gains == "distinct":
        gn = synth.norm_gains(d, inner, seed + 1)
    elif isinstance(gains, tuple):  # only the named gains; an "i" gain is shared by f and g
        g = synth.norm_gains(d, inner, seed + 1)
        gn = {k: g[k] for k in gains}
        if "i" in gn:
            gn["f"] = gn["g"] = gn["i"]
    L = oracle.make_layer(lat, gn, eps)
    dgains = None
    if gn is not None:
        dgains = {}
        cache = {}
        for k, v in gn.items():
            key = id(v)
            if key not in cache:
                cache[key] = dev(v, device)
            dgains[k] = cache[key]
    P = mmf.LayerParams.pack({k: dev(v, device) for k, v in lat.items()}, dgains, eps)
    return L, P


def check_layer_stages(L: "oracle.Layer", x: np.ndarray, h0, pr: dict, out_gpu: np.ndarray, act: str,
                       scan_rtol: float = 1e-4, shared: bool = True, decode: bool = False):
    """Stage-fed parity: every stage of the GPU layer against the oracle applied to the GPU's own stage inputs."""
    b, t, d = x.shape
    m = b * t
    eps = L.eps
    xf = x.reshape(m, d).astype(np.float32)
    rtol_out = 1e-4 if act == "f32" else 2e-2
    projs = [L.i, L.f, L.g]
    for q in range(1 if shared else 3):
        qq, ss, _ = oracle.quantize(xf, projs[q].gain, eps)
        assert_equal(pr["codes_x"][q], qq, "codes_x[%d]" % q)
        assert_equal(pr["scale_x"][q], ss, "scale_x[%d]" % q)
    acc = pr["acc_ifg"].reshape(m, 3, d)
    hat = []
    for q in range(3):
        src = 0 if shared else q
        ref = oracle.ternary_matmul(pr["codes_x"][src], projs[q].t)
        assert_equal(acc[:, q], ref, "acc_%s" % "ifg"[q])
        hat.append(oracle.dequant(ref, pr["scale_x"][src], projs[q].mu))
    f_ref, xt_ref = oracle.mixer_gates(hat[0], hat[1])
    assert_close(pr["f"], f_ref, 1e-4, "f")
    assert_close(pr["xt"], xt_ref, 1e-4, "xt")
    assert_close(pr["g"], hat[2], 1e-4, "g")
    h_ref = oracle.hgrn_scan(pr["xt"].reshape(b, t, d), pr["f"].reshape(b, t, d), h0)
    assert_close(pr["h"], h_ref.reshape(m, d), scan_rtol, "h")
    u_ref = oracle.gnorm_swish(pr["h"], pr["g"], L.g_norm_w, eps)
    assert_close(pr["u"], u_ref, 1e-4, "u")
    qq, ss, _ = oracle.quantize(pr["u"], L.o.gain, eps)
    assert_equal(pr["codes_u"], qq, "codes_u")
    assert_equal(pr["scale_u"], ss, "scale_u")
    acc_o = oracle.ternary_matmul(pr["codes_u"], L.o.t)
    assert_equal(pr["acc_o"], acc_o, "acc_o")
    x1_ref = xf.astype(np.float64) + oracle.dequant(acc_o, pr["scale_u"], L.o.mu)
    assert_close(pr["x1"], x1_ref, 1e-4, "x1")
    qq, ss, _ = oracle.quantize(pr["x1"], L.gate.gain, eps)
    assert_equal(pr["codes_x1"], qq, "codes_x1")
    assert_equal(pr["scale_x1"], ss, "scale_x1")
    acc_g = oracle.ternary_matmul(pr["codes_x1"], L.gate.t)
    assert_equal(pr["acc_gate"], acc_g, "acc_gate")
    ab = oracle.dequant(acc_g, pr["scale_x1"], L.gate.mu)
    inner = L.inner
    z_ref = oracle.silu(ab[:, :inner]) * ab[:, inner:]
    assert_close(pr["z"], z_ref, 1e-4, "z")
    qq, ss, _ = oracle.quantize(pr["z"], L.down.gain, eps)
    assert_equal(pr["codes_z"], qq, "codes_z")
    assert_equal(pr["scale_z"], ss, "scale_z")
    acc_dn = oracle.ternary_matmul(pr["codes_z"], L.down.t)
    assert_equal(pr["acc_down"], acc_dn, "acc_down")
    out_ref = pr["x1"].astype(np.float64) + oracle.dequant(acc_dn, pr["scale_z"], L.down.mu)
    assert_close(out_gpu.reshape(m, d), out_ref, rtol_out, "out")


def probe_rows(probe, rows) -> dict:
    """The probe's row-indexed stages for the given rows only (host arrays)."""
    import torch
    from ternary_weight_matmul_amd.binding import PROBE_FIELDS
    idx = torch.as_tensor(np.asarray(rows), device=probe.acc_ifg.device)
    out = {"codes_x": [t.index_select(0, idx).cpu().numpy() for t in probe.codes_x],
           "scale_x": [t.index_select(0, idx).cpu().numpy() for t in probe.scale_x]}
    for name in PROBE_FIELDS:
        out[name] = getattr(probe, name).index_select(0, idx).cpu().numpy()
    return out


def check_layer_sampled(L: "oracle.Layer", x: np.ndarray, h0, probe, out_gpu, act: str, b: int, t: int,
                        rows, chans, scan_rtol: float):
    """Stage-fed parity at full size on sampled tokens: every stage of the sampled rows against the
    oracle applied to the GPU's own stage inputs of those rows; the scan over the whole sequence of
    the sampled (sequence, channel) pairs, fed with the GPU's gate outputs of those channels."""
    import torch
    d = L.d
    eps = L.eps
    rows = np.asarray(sorted(rows))
    pr = probe_rows(probe, rows)
    xr = x.reshape(b * t, d)[rows].astype(np.float32)
    rtol_out = 1e-4 if act == "f32" else 2e-2
    projs = [L.i, L.f, L.g]
    qq, ss, _ = oracle.quantize(xr, L.i.gain, eps)
    assert_equal(pr["codes_x"][0], qq, "codes_x")
    assert_equal(pr["scale_x"][0], ss, "scale_x")
    acc = pr["acc_ifg"].reshape(len(rows), 3, d)
    hat = []
    for q in range(3):
        ref = oracle.ternary_matmul(pr["codes_x"][0], projs[q].t)
        assert_equal(acc[:, q], ref, "acc_%s" % "ifg"[q])
        hat.append(oracle.dequant(ref, pr["scale_x"][0], projs[q].mu))
    f_ref, xt_ref = oracle.mixer_gates(hat[0], hat[1])
    assert_close(pr["f"], f_ref, 1e-4, "f")
    assert_close(pr["xt"], xt_ref, 1e-4, "xt")
    assert_close(pr["g"], hat[2], 1e-4, "g")
    # the scan: whole sequences of the sampled channels
    for (bi, c) in chans:
        xs = probe.xt.view(b, t, d)[bi, :, c].cpu().numpy().reshape(1, t, 1)
        fs = probe.f.view(b, t, d)[bi, :, c].cpu().numpy().reshape(1, t, 1)
        hs = probe.h.view(b, t, d)[bi, :, c].cpu().numpy()
        h0c = None if h0 is None else np.asarray(h0)[bi, c].reshape(1, 1)
        assert_close(hs, oracle.hgrn_scan(xs, fs, h0c).reshape(t), scan_rtol, "h[%d,:,%d]" % (bi, c))
    u_ref = oracle.gnorm_swish(pr["h"], pr["g"], L.g_norm_w, eps)
    assert_close(pr["u"], u_ref, 1e-4, "u")
    qq, ss, _ = oracle.quantize(pr["u"], L.o.gain, eps)
    assert_equal(pr["codes_u"], qq, "codes_u")
    assert_equal(pr["scale_u"], ss, "scale_u")
    acc_o = oracle.ternary_matmul(pr["codes_u"], L.o.t)
    assert_equal(pr["acc_o"], acc_o, "acc_o")
    assert_close(pr["x1"], xr.astype(np.float64) + oracle.dequant(acc_o, pr["scale_u"], L.o.mu), 1e-4, "x1")
    qq, ss, _ = oracle.quantize(pr["x1"], L.gate.gain, eps)
    assert_equal(pr["codes_x1"], qq, "codes_x1")
    assert_equal(pr["scale_x1"], ss, "scale_x1")
    acc_g = oracle.ternary_matmul(pr["codes_x1"], L.gate.t)
    assert_equal(pr["acc_gate"], acc_g, "acc_gate")
    ab = oracle.dequant(acc_g, pr["scale_x1"], L.gate.mu)
    assert_close(pr["z"], oracle.silu(ab[:, :L.inner]) * ab[:, L.inner:], 1e-4, "z")
    qq, ss, _ = oracle.quantize(pr["z"], L.down.gain, eps)
    assert_equal(pr["codes_z"], qq, "codes_z")
    assert_equal(pr["scale_z"], ss, "scale_z")
    acc_dn = oracle.ternary_matmul(pr["codes_z"], L.down.t)
    assert_equal(pr["acc_down"], acc_dn, "acc_down")
    out_rows = host(out_gpu.reshape(b * t, d).index_select(0, torch.as_tensor(rows, device=out_gpu.device)))
    out_ref = pr["x1"].astype(np.float64) + oracle.dequant(acc_dn, pr["scale_z"], L.down.mu)
    assert_close(out_rows, out_ref, rtol_out, "out")
