"""C-ABI contract checks that run without a GPU.

The library must load, export every entry point include/mmf.h declares, and
reject bad arguments on the host -- with a status code and a message --
before it makes any HIP call. Fake device addresses are used only where
validation fails before they could be touched.
"""
import ctypes
import os
import re
import subprocess

import pytest

import ternary_weight_matmul_amd as mmf
from ternary_weight_matmul_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 0x7f0000000000  # 256-byte aligned, never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libmmf.so not built")
    return mmf.load()


def _declared():
    text = open(os.path.join(ROOT, "include", "mmf.h")).read()
    return sorted(set(re.findall(r"\b(mmf_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared() == sorted(B.SYMBOLS)


def test_every_declared_symbol_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (mmf_[a-z_0-9]+)", out))
    for name in _declared():
        assert name in exported, name
        assert hasattr(lib, name)


def _weight(n=64, k=64, packed=FAKE, mu=FAKE + 4096, norm=None):
    return B.CTernaryWeight(packed, mu, norm, n, k)


def _layer(d=64, inner=96):
    w = lambda n, k: _weight(n, k)  # noqa: E731
    return B.CLayerWeights(w(d, d), w(d, d), w(d, d), w(d, d), w(2 * inner, d), w(d, inner), None, d, inner, 1e-8)


def _err(lib):
    return lib.mmf_last_error().decode()


def test_pack_validation(lib):
    sz = ctypes.c_size_t(0)
    assert lib.mmf_ternary_pack_workspace_size(8, 20, ctypes.byref(sz)) == UNSUPPORTED
    assert "multiple of 16" in _err(lib)
    assert lib.mmf_ternary_pack_workspace_size(0, 32, ctypes.byref(sz)) == INVALID
    assert lib.mmf_ternary_pack_workspace_size(8, 32, ctypes.byref(sz)) == OK and sz.value > 0
    assert lib.mmf_ternary_pack(None, 8, 32, FAKE, FAKE, FAKE, sz.value, None) == INVALID
    assert lib.mmf_ternary_pack(FAKE, 8, 32, FAKE, FAKE, FAKE, sz.value - 1, None) == WORKSPACE
    assert lib.mmf_ternary_pack(FAKE + 4, 8, 32, FAKE, FAKE, FAKE, sz.value, None) == INVALID


def test_bitlinear_validation(lib):
    sz = ctypes.c_size_t(0)
    assert lib.mmf_bitlinear_workspace_size(16, 64, ctypes.byref(sz)) == OK
    need = sz.value
    assert need >= 16 * 64 + 16 * 8
    w = _weight()
    args = lambda **kw: dict(dict(x=FAKE, xt=0, m=16, w=ctypes.byref(w), eps=1e-8, y=FAKE, yt=0, c=None, s=None,  # noqa: E731
                                  a=None, ws=FAKE, wsb=need, st=None), **kw)

    def call(**kw):
        a = args(**kw)
        return lib.mmf_bitlinear_fwd(a["x"], a["xt"], a["m"], a["w"], ctypes.c_float(a["eps"]), a["y"], a["yt"],
                                     a["c"], a["s"], a["a"], a["ws"], a["wsb"], a["st"])
    assert call(w=None) == INVALID
    assert call(xt=7) == INVALID
    assert call(m=-1) == INVALID
    assert call(x=None) == INVALID
    assert call(wsb=need - 1) == WORKSPACE
    assert call(ws=FAKE + 16) == WORKSPACE
    assert call(eps=-1.0) == INVALID
    bad = _weight(k=40)
    assert call(w=ctypes.byref(bad)) == UNSUPPORTED
    big = _weight(k=65536 + 16)
    assert call(w=ctypes.byref(big)) == UNSUPPORTED
    nomu = _weight(mu=None)
    assert call(w=ctypes.byref(nomu)) == INVALID
    # m == 0 is valid and launches nothing
    assert call(m=0, x=None, y=None, ws=None, wsb=0) == OK
    assert lib.mmf_last_path().decode() == "empty"


def test_scan_validation(lib):
    sz = ctypes.c_size_t(0)
    assert lib.mmf_hgrn_scan_workspace_size(2, 10, 0, 0, ctypes.byref(sz)) == INVALID
    assert lib.mmf_hgrn_scan_workspace_size(2, 10, 64, 9, ctypes.byref(sz)) == INVALID
    assert lib.mmf_hgrn_scan_workspace_size(1, 4096, 64, 1, ctypes.byref(sz)) == OK and sz.value == 0
    assert lib.mmf_hgrn_scan_workspace_size(1, 4096, 64, 2, ctypes.byref(sz)) == OK and sz.value > 0
    assert lib.mmf_hgrn_scan_fwd(None, FAKE, None, FAKE, None, 1, 4, 64, 1, None, 0, None) == INVALID
    assert lib.mmf_hgrn_scan_fwd(FAKE, FAKE, None, FAKE, None, 1, 4096, 64, 2, None, 0, None) == WORKSPACE


def test_hgrn2_scan_validation(lib):
    """mmf_hgrn2_scan_fwd rejects unsupported head widths, ragged heads, missing and aliased
    buffers on the host."""
    F = [FAKE + k * (1 << 24) for k in range(6)]
    f, i, o, s0, y, sl = F

    def h2(*a, mode=0):
        return lib.mmf_hgrn2_scan_fwd(*a[:10], mode, a[10])
    assert h2(f, i, o, s0, y, sl, 1, 4, 256, 64, None, mode=7) == INVALID
    assert h2(f, i, o, s0, y, sl, 1, 4, 256, 32, None, mode=2) == UNSUPPORTED  # chunked: heads of 64 or 128
    assert h2(f, i, o, s0, y, sl, 1, 4, 256, 48, None) == UNSUPPORTED
    assert h2(f, i, o, s0, y, sl, 1, 4, 256, 8, None) == UNSUPPORTED
    assert h2(f, i, o, s0, y, sl, 1, 4, 96, 64, None) == INVALID
    assert h2(f, i, o, s0, y, sl, -1, 4, 256, 64, None) == INVALID
    assert h2(None, i, o, s0, y, sl, 1, 4, 256, 64, None) == INVALID
    assert h2(f, i, o, s0, None, sl, 1, 4, 256, 64, None) == INVALID
    assert h2(f, i, o, s0, i, sl, 1, 4, 256, 64, None) == INVALID   # y aliases i
    assert h2(f, i, o, s0, y, f, 1, 4, 256, 64, None) == INVALID   # s_last aliases f
    assert h2(f, i, o, s0, y, y, 1, 4, 256, 64, None) == INVALID   # s_last aliases y
    assert "alias" in B.last_error()
    assert h2(f + 4, i, o, s0, y, sl, 1, 4, 256, 64, None) == INVALID  # misaligned
    assert h2(f, i, o, s0, y, sl, 0, 4, 256, 64, None) == OK       # nothing to do
    # the chunked form addresses a sequence with 32-bit byte offsets: (t + 32) * d * 4 < 2^31
    t_max = (2 ** 31 - 1) // 4 // 2048 - 32
    assert h2(f, i, o, s0, y, sl, 1, t_max + 1, 2048, 128, None, mode=2) == UNSUPPORTED
    assert "2 GiB" in B.last_error()
    assert h2(f, i, o, s0, y, sl, 0, t_max, 2048, 128, None, mode=2) == OK


def test_bitlinear_bwd_validation(lib):
    sz = ctypes.c_size_t(0)
    w = _weight(64, 128)
    assert lib.mmf_bitlinear_bwd_workspace_size(32, ctypes.byref(w), 0, ctypes.byref(sz)) == OK
    f32_need = sz.value
    assert lib.mmf_bitlinear_bwd_workspace_size(32, ctypes.byref(w), 1, ctypes.byref(sz)) == OK
    assert f32_need > sz.value > 0  # an fp32 dy needs a bf16 copy
    assert lib.mmf_bitlinear_bwd_workspace_size(-1, ctypes.byref(w), 1, ctypes.byref(sz)) == INVALID
    x, dy, dx, dw, dg, ws = (FAKE + 65536 * i for i in range(6))
    call = lib.mmf_bitlinear_bwd
    big = 1 << 30
    assert call(None, 1, 32, ctypes.byref(w), 1e-8, dy, 1, dx, 1, dw, dg, ws, big, None) == INVALID
    assert call(x, 1, 32, ctypes.byref(w), -1.0, dy, 1, dx, 1, dw, dg, ws, big, None) == INVALID
    assert call(x, 1, 32, ctypes.byref(w), 1e-8, dy, 1, dx, 1, dw, dg, ws, 16, None) == WORKSPACE
    odd = _weight(60, 128)
    assert call(x, 1, 32, ctypes.byref(odd), 1e-8, dy, 1, dx, 1, dw, dg, ws, big, None) == UNSUPPORTED
    wide = _weight(64, 8192 + 16)
    assert call(x, 1, 32, ctypes.byref(wide), 1e-8, dy, 1, dx, 1, dw, dg, ws, big, None) == UNSUPPORTED


def test_generation_validation(lib):
    ids, table, out, x, tok, ws = (FAKE + 65536 * i for i in range(6))
    assert lib.mmf_embed(ids, 4, table, 1, 1000, 0, out, None) == INVALID          # d = 0
    assert lib.mmf_embed(ids, 4, table, 1, 1000, 4, out, None) == UNSUPPORTED      # 8-byte rows
    assert lib.mmf_embed(None, 4, table, 1, 1000, 64, out, None) == INVALID
    assert lib.mmf_embed(None, 0, None, 1, 1000, 64, None, None) == OK             # nothing to do
    sz = ctypes.c_size_t(0)
    head = _weight(1000, 256)
    assert lib.mmf_greedy_head_workspace_size(8, ctypes.byref(head), ctypes.byref(sz)) == OK and sz.value > 0
    odd = _weight(1002, 256)
    big = 1 << 30
    assert lib.mmf_greedy_head(x, 1, 8, ctypes.byref(odd), 1e-8, tok, None, ws, big, None) == UNSUPPORTED
    assert lib.mmf_greedy_head(x, 1, 8, ctypes.byref(head), 1e-8, None, None, ws, big, None) == INVALID
    assert lib.mmf_greedy_head(x, 1, 8, ctypes.byref(head), 1e-8, tok, None, ws, 16, None) == WORKSPACE


def test_scan_bwd_validation(lib):
    f, h, dh, dx, df, h0, gl, dh0 = (FAKE + 256 * i for i in range(8))
    call = lib.mmf_hgrn_scan_bwd
    assert call(None, h, h0, dh, gl, dx, df, dh0, 1, 4, 64, 1, None) == INVALID  # f missing
    assert call(f, h, h0, dh, gl, None, df, dh0, 1, 4, 64, 1, None) == INVALID   # dx missing
    assert call(f, h, h0, dh, gl, dx, df, dh0, 1, 4, 0, 1, None) == INVALID      # d = 0
    assert call(f, h, h0, dh, gl, dx, df, dh0, 1, 4, 64, 7, None) == INVALID     # mode
    assert call(f, h, h0, dh, gl, dx, h, dh0, 1, 4, 64, 1, None) == INVALID      # df aliases h
    assert call(f, h, h0, dh, gl, dx, df, gl, 1, 4, 64, 1, None) == INVALID      # dh0 aliases dh_last
    assert call(f, h, h0, dh, gl, f, df, dh0, 1, 4, 64, 1, None) == INVALID      # dx aliases f
    assert "alias" in _err(lib)
    # no sequences: valid, nothing launched
    assert call(None, None, None, None, None, None, None, None, 0, 4, 64, 0, None) == OK


def test_layer_validation(lib):
    L = _layer()
    sz = ctypes.c_size_t(0)
    assert lib.mmf_layer_workspace_size(ctypes.byref(L), 2, 8, ctypes.byref(sz)) == OK
    need = sz.value
    assert need > 0
    bad = _layer()
    bad.gate = _weight(96, 64)  # must be [2*inner][d]
    assert lib.mmf_layer_workspace_size(ctypes.byref(bad), 2, 8, ctypes.byref(sz)) == INVALID
    assert "gate_proj" in _err(lib)
    odd = _layer(d=72)
    assert lib.mmf_layer_workspace_size(ctypes.byref(odd), 2, 8, ctypes.byref(sz)) == UNSUPPORTED
    wide = _layer(d=8192 + 16)
    assert lib.mmf_layer_workspace_size(ctypes.byref(wide), 1, 1, ctypes.byref(sz)) == UNSUPPORTED
    assert lib.mmf_layer_fwd(ctypes.byref(L), FAKE, FAKE, 0, 2, 8, None, None, 0, FAKE, need - 1, None, None) == WORKSPACE
    assert lib.mmf_layer_fwd(ctypes.byref(L), FAKE, FAKE, 5, 2, 8, None, None, 0, FAKE, need, None, None) == INVALID
    assert lib.mmf_layer_fwd(ctypes.byref(L), FAKE, FAKE, 0, 2, 8, None, None, 7, FAKE, need, None, None) == INVALID
    assert lib.mmf_layer_fwd(ctypes.byref(L), FAKE + 8, FAKE, 0, 2, 8, None, None, 0, FAKE, need, None, None) == INVALID
    assert lib.mmf_layer_decode_step(ctypes.byref(L), FAKE, FAKE, 0, 2, None, FAKE, need, None, None) == INVALID
    assert lib.mmf_layer_workspace_size(ctypes.byref(L), 4, 1, ctypes.byref(sz)) == OK
    assert lib.mmf_layer_decode_step(ctypes.byref(L), FAKE, FAKE, 0, 4, FAKE, FAKE, sz.value - 256, None, None) == WORKSPACE


def test_workspace_grows_with_tokens(lib):
    L = _layer()
    sizes = []
    for t in (1, 16, 256):
        sz = ctypes.c_size_t(0)
        assert lib.mmf_layer_workspace_size(ctypes.byref(L), 2, t, ctypes.byref(sz)) == OK
        sizes.append(sz.value)
    assert sizes[0] < sizes[1] < sizes[2]
    # distinct i/f/g gains need three quantised copies of x
    L2 = _layer()
    L2.f.norm_w = FAKE + 8192
    sz2 = ctypes.c_size_t(0)
    assert lib.mmf_layer_workspace_size(ctypes.byref(L2), 2, 256, ctypes.byref(sz2)) == OK
    assert sz2.value > sizes[2]


def test_decode_kernel_modes(lib):
    """mmf_set_decode_kernel accepts auto / separate and rejects the rest without touching the GPU."""
    try:
        for mode in (0, 1):
            assert lib.mmf_set_decode_kernel(mode) == OK
        for mode in (-1, 2, 3, 99):
            assert lib.mmf_set_decode_kernel(mode) == INVALID
            assert b"decode kernel mode" in lib.mmf_last_error()
    finally:
        lib.mmf_set_decode_kernel(0)
    for name, mode in B.DECODE_KERNELS.items():
        B.set_decode_kernel(name)
    B.set_decode_kernel("auto")


def test_hbm_ceiling_rejects_bad_arguments(lib):
    """mmf_hbm_ceiling validates on the host before any HIP call."""
    import ctypes as C
    p = C.c_void_p(FAKE)
    q = C.c_void_p(FAKE + (1 << 30))
    assert lib.mmf_hbm_ceiling(3, p, q, 4096, None) == INVALID
    assert lib.mmf_hbm_ceiling(0, p, q, 4100, None) == INVALID
    assert lib.mmf_hbm_ceiling(1, p, C.c_void_p(FAKE + 8), 4096, None) == INVALID  # overlap
    assert lib.mmf_hbm_ceiling(2, p, C.c_void_p(FAKE + 4096), 4096, None) == INVALID  # overlaps the second source
    assert lib.mmf_hbm_ceiling(1, None, q, 4096, None) == INVALID


def test_stack_decode_validation(lib):
    SZ = ctypes.c_size_t
    n = 3
    layers = (B.CLayerWeights * n)(*[_layer(256, 512) for _ in range(n)])
    need = SZ(0)
    assert lib.mmf_stack_decode_workspace_size(layers, n, 16, ctypes.byref(need)) == OK
    assert need.value > 0
    big = SZ(0)
    assert lib.mmf_stack_decode_workspace_size(layers, n, 8, ctypes.byref(big)) == OK and big.value < need.value
    # batch outside 1..16, widths that are not multiples of 256, no blocks
    assert lib.mmf_stack_decode_workspace_size(layers, n, 17, ctypes.byref(need)) == UNSUPPORTED
    assert "1..16" in _err(lib)
    assert lib.mmf_stack_decode_workspace_size(layers, n, 0, ctypes.byref(need)) == UNSUPPORTED
    odd = (B.CLayerWeights * 1)(_layer(64, 96))
    assert lib.mmf_stack_decode_workspace_size(odd, 1, 4, ctypes.byref(need)) == UNSUPPORTED
    assert "256" in _err(lib)
    assert lib.mmf_stack_decode_workspace_size(layers, 0, 4, ctypes.byref(need)) == INVALID
    assert lib.mmf_stack_decode_workspace_size(None, 1, 4, ctypes.byref(need)) == INVALID
    # blocks of different widths; i/f/g with different gains
    mixed = (B.CLayerWeights * 2)(_layer(256, 512), _layer(512, 512))
    assert lib.mmf_stack_decode_workspace_size(mixed, 2, 4, ctypes.byref(need)) == INVALID
    split = _layer(256, 512)
    split.f.norm_w = FAKE + 8192
    gains = (B.CLayerWeights * 1)(split)
    assert lib.mmf_stack_decode_workspace_size(gains, 1, 4, ctypes.byref(need)) == UNSUPPORTED
    # bind: no states, a NULL state, a short workspace; step: aliasing, bad dtype, short workspace
    assert lib.mmf_stack_decode_workspace_size(layers, n, 4, ctypes.byref(need)) == OK
    hs = (ctypes.c_void_p * n)(FAKE, None, FAKE)
    assert lib.mmf_stack_decode_bind(layers, n, 4, None, FAKE, need.value, None) == INVALID
    assert lib.mmf_stack_decode_bind(layers, n, 4, hs, FAKE, need.value, None) == INVALID
    assert lib.mmf_stack_decode_bind(layers, n, 4, hs, FAKE, need.value - 1, None) == WORKSPACE
    assert lib.mmf_stack_decode_step(layers, n, FAKE, FAKE, 0, 4, FAKE, need.value, None) == INVALID
    assert "overlap" in _err(lib)
    assert lib.mmf_stack_decode_step(layers, n, FAKE, FAKE + 65536, 7, 4, FAKE, need.value, None) == INVALID
    assert lib.mmf_stack_decode_step(layers, n, FAKE, FAKE + 65536, 0, 4, FAKE, 256, None) == WORKSPACE
    assert lib.mmf_stack_decode_expired(None) == INVALID


def test_mfma_ceiling_rejects_bad_arguments(lib):
    ops = ctypes.c_int64(0)
    assert lib.mmf_mfma_ceiling(0, FAKE, 1 << 20, ctypes.byref(ops), None) == INVALID
    assert lib.mmf_mfma_ceiling(10, None, 1 << 20, ctypes.byref(ops), None) == INVALID
    assert lib.mmf_mfma_ceiling(10, FAKE, 1 << 20, None, None) == INVALID
