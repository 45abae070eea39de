"""ctypes binding of libmmf.so (the C ABI in include/mmf.h).

Argument marshalling only: tensors are passed as device pointers with the
current torch stream; every step of the computation runs in the HIP kernels.
There is no fallback: if the library is missing or a call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# MMF_LIB: another build of the same sources (the host-sanitizer check loads one)
LIB_PATH = os.environ.get("MMF_LIB") or os.path.join(_HERE, "libmmf.so")

__all__ = [
    "MMFError", "load", "LIB_PATH", "SYMBOLS", "PackedLinear", "LayerParams", "LayerProbe",
    "ternary_pack", "bitlinear_fwd", "bitlinear_bwd", "embed", "greedy_head", "hgrn_scan_fwd", "hgrn_scan_bwd",
    "hgrn2_scan_fwd", "layer_fwd", "layer_bwd",
    "layer_decode_step", "layer_decode_step_noalloc",
    "layer_workspace_size", "last_path", "last_error", "SCAN_MODES", "timing_enable", "timing_collect",
    "StackDecoder", "stack_decode_expired",
    "set_decode_kernel", "DECODE_KERNELS", "hbm_ceiling", "mfma_ceiling",
]

# Every entry point declared in include/mmf.h.
SYMBOLS = [
    "mmf_last_error", "mmf_last_path",
    "mmf_ternary_pack_workspace_size", "mmf_ternary_pack",
    "mmf_bitlinear_workspace_size", "mmf_bitlinear_fwd",
    "mmf_bitlinear_bwd_workspace_size", "mmf_bitlinear_bwd",
    "mmf_embed", "mmf_greedy_head_workspace_size", "mmf_greedy_head",
    "mmf_hgrn_scan_workspace_size", "mmf_hgrn_scan_fwd", "mmf_hgrn_scan_bwd", "mmf_hgrn2_scan_fwd",
    "mmf_layer_workspace_size", "mmf_layer_fwd", "mmf_layer_decode_step", "mmf_layer_decode_step_noalloc",
    "mmf_layer_bwd_workspace_size", "mmf_layer_bwd",
    "mmf_set_decode_kernel",
    "mmf_stack_decode_workspace_size", "mmf_stack_decode_bind", "mmf_stack_decode_step", "mmf_stack_decode_expired",
    "mmf_timing_enable", "mmf_timing_collect", "mmf_hbm_ceiling", "mmf_mfma_ceiling",
]

SCAN_MODES = {"auto": 0, "recurrent": 1, "chunk": 2}
STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "WORKSPACE", 4: "HIP"}


class MMFError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (STATUS.get(status, status), msg))
        self.status = status


P = ctypes.c_void_p
I32, I64, F32, SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class CTernaryWeight(ctypes.Structure):
    _fields_ = [("packed", P), ("mu", P), ("norm_w", P), ("n", I32), ("k", I32)]


class CLayerWeights(ctypes.Structure):
    _fields_ = [("i", CTernaryWeight), ("f", CTernaryWeight), ("g", CTernaryWeight),
                ("o", CTernaryWeight), ("gate", CTernaryWeight), ("down", CTernaryWeight),
                ("g_norm_w", P), ("d", I32), ("inner", I32), ("eps", F32)]


PROBE_FIELDS = ["acc_ifg", "f", "xt", "g", "h", "u", "codes_u", "scale_u", "acc_o", "x1",
                "codes_x1", "scale_x1", "acc_gate", "z", "codes_z", "scale_z", "acc_down"]


class CKernelTiming(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char * 40), ("m", I64), ("n", I32), ("k", I32), ("ms", F32)]


class CLayerGrads(ctypes.Structure):
    _fields_ = [("dx", P), ("dh0", P), ("dw", P * 6), ("dgain", P * 6), ("dg_norm_w", P)]


class CLayerProbe(ctypes.Structure):
    _fields_ = [("codes_x", P * 3), ("scale_x", P * 3)] + [(n, P) for n in PROBE_FIELDS]


_lib = None


def load():
    """Open libmmf.so (built by ternary_weight_matmul_amd/build.py); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libmmf.so not built at %s (run __graft_entry__.build())" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    lib.mmf_last_error.restype = ctypes.c_char_p
    lib.mmf_last_path.restype = ctypes.c_char_p
    lib.mmf_ternary_pack_workspace_size.argtypes = [I32, I32, ctypes.POINTER(SZ)]
    lib.mmf_ternary_pack.argtypes = [P, I32, I32, P, P, P, SZ, P]
    lib.mmf_bitlinear_workspace_size.argtypes = [I64, I32, ctypes.POINTER(SZ)]
    lib.mmf_bitlinear_fwd.argtypes = [P, ctypes.c_int, I64, ctypes.POINTER(CTernaryWeight), F32, P,
                                      ctypes.c_int, P, P, P, P, SZ, P]
    lib.mmf_bitlinear_bwd_workspace_size.argtypes = [I64, ctypes.POINTER(CTernaryWeight), ctypes.c_int,
                                                     ctypes.POINTER(SZ)]
    lib.mmf_bitlinear_bwd.argtypes = [P, ctypes.c_int, I64, ctypes.POINTER(CTernaryWeight), F32, P, ctypes.c_int,
                                      P, ctypes.c_int, P, P, P, SZ, P]
    lib.mmf_embed.argtypes = [P, I64, P, ctypes.c_int, I64, I32, P, P]
    lib.mmf_greedy_head_workspace_size.argtypes = [I64, ctypes.POINTER(CTernaryWeight), ctypes.POINTER(SZ)]
    lib.mmf_greedy_head.argtypes = [P, ctypes.c_int, I64, ctypes.POINTER(CTernaryWeight), F32, P, P, P, SZ, P]
    lib.mmf_hgrn_scan_workspace_size.argtypes = [I64, I64, I64, ctypes.c_int, ctypes.POINTER(SZ)]
    lib.mmf_hgrn_scan_fwd.argtypes = [P, P, P, P, P, I64, I64, I64, ctypes.c_int, P, SZ, P]
    lib.mmf_hgrn_scan_bwd.argtypes = [P, P, P, P, P, P, P, P, I64, I64, I64, ctypes.c_int, P]
    lib.mmf_hgrn2_scan_fwd.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, ctypes.c_int, P]
    lib.mmf_layer_workspace_size.argtypes = [ctypes.POINTER(CLayerWeights), I64, I64, ctypes.POINTER(SZ)]
    lib.mmf_layer_fwd.argtypes = [ctypes.POINTER(CLayerWeights), P, P, ctypes.c_int, I64, I64, P, P,
                                  ctypes.c_int, P, SZ, ctypes.POINTER(CLayerProbe), P]
    lib.mmf_layer_decode_step.argtypes = [ctypes.POINTER(CLayerWeights), P, P, ctypes.c_int, I64, P, P, SZ,
                                          ctypes.POINTER(CLayerProbe), P]
    lib.mmf_layer_decode_step_noalloc.argtypes = [ctypes.POINTER(CLayerWeights), P, P, ctypes.c_int, I64, P,
                                                  ctypes.POINTER(CLayerProbe), P]
    lib.mmf_layer_bwd_workspace_size.argtypes = [ctypes.POINTER(CLayerWeights), I64, I64, ctypes.POINTER(SZ)]
    lib.mmf_layer_bwd.argtypes = [ctypes.POINTER(CLayerWeights), P, P, ctypes.c_int, I64, I64, P, P, ctypes.c_int,
                                  ctypes.POINTER(CLayerGrads), P, SZ, P]
    lib.mmf_set_decode_kernel.argtypes = [ctypes.c_int]
    lib.mmf_stack_decode_workspace_size.argtypes = [ctypes.POINTER(CLayerWeights), I32, I64, ctypes.POINTER(SZ)]
    lib.mmf_stack_decode_bind.argtypes = [ctypes.POINTER(CLayerWeights), I32, I64, ctypes.POINTER(P), P, SZ, P]
    lib.mmf_stack_decode_step.argtypes = [ctypes.POINTER(CLayerWeights), I32, P, P, ctypes.c_int, I64, P, SZ, P]
    lib.mmf_stack_decode_expired.argtypes = [ctypes.POINTER(ctypes.c_uint32)]
    lib.mmf_timing_enable.argtypes = [ctypes.c_int]
    lib.mmf_timing_collect.argtypes = [ctypes.POINTER(CKernelTiming), I32, ctypes.POINTER(I32)]
    lib.mmf_hbm_ceiling.argtypes = [ctypes.c_int, P, P, I64, P]
    lib.mmf_mfma_ceiling.argtypes = [I64, P, I64, ctypes.POINTER(I64), P]
    for name in SYMBOLS[2:]:
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def last_error() -> str:
    return load().mmf_last_error().decode()


def last_path() -> str:
    return load().mmf_last_path().decode()


DECODE_KERNELS = {"auto": 0, "separate": 1}


def set_decode_kernel(mode: str = "auto"):
    """Implementation of layer_decode_step, process-wide (mmf_set_decode_kernel)."""
    _check(load().mmf_set_decode_kernel(DECODE_KERNELS[mode]))


def timing_enable(on: bool = True):
    """Bracket every kernel launch of this thread's library calls with HIP events (measurement only)."""
    _check(load().mmf_timing_enable(1 if on else 0))


def timing_collect() -> list:
    """[(kernel, m, n, k, ms)] for every launch recorded since timing_enable(True)."""
    lib = load()
    count = I32(0)
    _check(lib.mmf_timing_collect(None, 0, ctypes.byref(count)))
    recs = (CKernelTiming * max(count.value, 1))()
    _check(lib.mmf_timing_collect(recs, count.value, ctypes.byref(count)))
    return [(r.kernel.decode(), r.m, r.n, r.k, r.ms) for r in recs[:count.value]]


def hbm_ceiling(src, dst, mode: str = "read"):
    """Measured HBM roof (mmf_hbm_ceiling): "read" streams src (dst: a sink of at least 32768
    bytes); "copy" copies src into dst; "2r1w" writes dst = first half of src ^ second half
    (src twice dst's size)."""
    n = src.numel() * src.element_size()
    m = {"read": 0, "copy": 1, "2r1w": 2}[mode]
    _check(load().mmf_hbm_ceiling(m, _ptr(src), _ptr(dst), n // 2 if m == 2 else n, _stream()))


def mfma_ceiling(iters: int, sink) -> int:
    """Measured int8 MFMA roof (mmf_mfma_ceiling): launches the MFMA-only loop on the current
    stream with `sink` (a device buffer of at least 4 * CUs uint32) and returns the operations
    the launch performs; time it with events around the call."""
    ops = I64(0)
    _check(load().mmf_mfma_ceiling(iters, _ptr(sink), sink.numel() * sink.element_size(), ctypes.byref(ops),
                                   _stream()))
    return ops.value


def _check(status: int):
    if status != 0:
        raise MMFError(status, last_error())


def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream():
    torch = _torch()
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.float32:
        return 0
    if dt == torch.bfloat16:
        return 1
    raise TypeError("activation dtype must be float32 or bfloat16, got %s" % dt)


def _workspace(nbytes: int, device, ws=None):
    torch = _torch()
    if ws is not None and ws.numel() >= nbytes:
        return ws
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


@dataclass
class PackedLinear:
    """A packed ternary weight on the device: words [n, k/16] (int32 storage), mu [1], RMSNorm gain [k] or None."""
    packed: object
    mu: object
    norm_w: Optional[object]
    n: int
    k: int

    def c(self) -> CTernaryWeight:
        return CTernaryWeight(_ptr(self.packed), _ptr(self.mu), _ptr(self.norm_w), self.n, self.k)


def ternary_pack(w, norm_w=None) -> PackedLinear:
    """Ternarise and pack a latent fp32 weight [n, k] on the device (mmf_ternary_pack)."""
    torch = _torch()
    lib = load()
    if w.dtype != torch.float32 or w.dim() != 2 or not w.is_contiguous():
        raise TypeError("w must be a contiguous 2-d float32 tensor")
    n, k = w.shape
    need = SZ(0)
    _check(lib.mmf_ternary_pack_workspace_size(n, k, ctypes.byref(need)))
    packed = torch.empty((n, k // 16), dtype=torch.int32, device=w.device)
    mu = torch.empty(1, dtype=torch.float32, device=w.device)
    ws = _workspace(need.value, w.device)
    _check(lib.mmf_ternary_pack(_ptr(w), n, k, _ptr(packed), _ptr(mu), _ptr(ws), need.value, _stream()))
    return PackedLinear(packed, mu, norm_w, n, k)


def bitlinear_fwd(x, w: PackedLinear, eps: float = 1e-8, out_dtype=None, codes_out=None, scale_out=None,
                  acc_out=None, ws=None):
    """FusedBitLinear on rows of x [..., k] (mmf_bitlinear_fwd); returns y [..., n]."""
    torch = _torch()
    lib = load()
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    k = x.shape[-1]
    m = x.numel() // k if k else 0
    out_dtype = out_dtype or x.dtype
    y = torch.empty(x.shape[:-1] + (w.n,), dtype=out_dtype, device=x.device)
    need = SZ(0)
    _check(lib.mmf_bitlinear_workspace_size(m, k, ctypes.byref(need)))
    ws = _workspace(need.value, x.device, ws)
    cw = w.c()
    _check(lib.mmf_bitlinear_fwd(_ptr(x), _dtype_code(x.dtype), m, ctypes.byref(cw), F32(eps), _ptr(y),
                                 _dtype_code(out_dtype), _ptr(codes_out), _ptr(scale_out), _ptr(acc_out),
                                 _ptr(ws), ws.numel(), _stream()))
    return y


def bitlinear_bwd(x, w: PackedLinear, dy, eps: float = 1e-8, want_dx=True, want_dw=True, want_dgain=False,
                  dx_dtype=None, ws=None):
    """Derivative of FusedBitLinear with straight-through quantisers (mmf_bitlinear_bwd):
    x [m, k] (the forward's input), dy [m, n]; returns (dx [m, k] or None, dw [n, k] fp32 or None,
    dgain [k] fp32 or None)."""
    torch = _torch()
    lib = load()
    if not x.is_contiguous() or not dy.is_contiguous():
        raise ValueError("x and dy must be contiguous")
    k = x.shape[-1]
    m = x.numel() // k if k else 0
    if dy.shape[-1] != w.n or dy.numel() != m * w.n:
        raise ValueError("dy must be [m, n]")
    dx = torch.empty(x.shape, dtype=dx_dtype or x.dtype, device=x.device) if want_dx else None
    dw = torch.empty((w.n, k), dtype=torch.float32, device=x.device) if want_dw else None
    dgain = torch.empty((k,), dtype=torch.float32, device=x.device) if want_dgain else None
    cw = w.c()
    need = SZ(0)
    _check(lib.mmf_bitlinear_bwd_workspace_size(m, ctypes.byref(cw), _dtype_code(dy.dtype), ctypes.byref(need)))
    ws = _workspace(need.value, x.device, ws)
    _check(lib.mmf_bitlinear_bwd(_ptr(x), _dtype_code(x.dtype), m, ctypes.byref(cw), F32(eps), _ptr(dy),
                                 _dtype_code(dy.dtype), _ptr(dx), _dtype_code(dx.dtype if dx is not None else x.dtype),
                                 _ptr(dw), _ptr(dgain), _ptr(ws), ws.numel(), _stream()))
    return dx, dw, dgain


def embed(ids, table, out=None):
    """Rows of an embedding table [vocab, d] (fp32 or bf16) for int32 token ids (mmf_embed);
    ids outside [0, vocab) give zero rows."""
    torch = _torch()
    lib = load()
    if ids.dtype != torch.int32 or not ids.is_contiguous() or not table.is_contiguous() or table.dim() != 2:
        raise TypeError("ids must be contiguous int32 and table a contiguous [vocab, d] tensor")
    vocab, d = table.shape
    out = out if out is not None else torch.empty((ids.numel(), d), dtype=table.dtype, device=table.device)
    _check(lib.mmf_embed(_ptr(ids), ids.numel(), _ptr(table), _dtype_code(table.dtype), vocab, d, _ptr(out),
                         _stream()))
    return out


def greedy_head(x, head: PackedLinear, eps: float = 1e-8, tokens=None, logits=None, ws=None):
    """Next token of each row of x [b, k] from a FusedBitLinear head (mmf_greedy_head): the smallest
    id of the largest exact sum. Returns tokens [b] int32 (logits [b, vocab] fp32 filled if given)."""
    torch = _torch()
    lib = load()
    if not x.is_contiguous() or x.dim() != 2:
        raise ValueError("x must be a contiguous [b, k] tensor")
    b = x.shape[0]
    tokens = tokens if tokens is not None else torch.empty((b,), dtype=torch.int32, device=x.device)
    cw = head.c()
    need = SZ(0)
    _check(lib.mmf_greedy_head_workspace_size(b, ctypes.byref(cw), ctypes.byref(need)))
    ws = _workspace(need.value, x.device, ws)
    _check(lib.mmf_greedy_head(_ptr(x), _dtype_code(x.dtype), b, ctypes.byref(cw), F32(eps), _ptr(tokens),
                               _ptr(logits), _ptr(ws), ws.numel(), _stream()))
    return tokens


def hgrn_scan_fwd(x, f, h0=None, mode: str = "auto", out=None, h_last=None, ws=None):
    """h_t = f_t * h_{t-1} + x_t over x, f [b, t, d] fp32 (mmf_hgrn_scan_fwd); returns h."""
    torch = _torch()
    lib = load()
    if x.shape != f.shape or x.dim() != 3:
        raise ValueError("x and f must both be [b, t, d]")
    for t_ in (x, f):
        if t_.dtype != torch.float32 or not t_.is_contiguous():
            raise TypeError("x and f must be contiguous float32")
    b, t, d = x.shape
    h = out if out is not None else torch.empty_like(x)
    need = SZ(0)
    _check(lib.mmf_hgrn_scan_workspace_size(b, t, d, SCAN_MODES[mode], ctypes.byref(need)))
    wsb = _workspace(need.value, x.device, ws)
    _check(lib.mmf_hgrn_scan_fwd(_ptr(x), _ptr(f), _ptr(h0), _ptr(h), _ptr(h_last), b, t, d, SCAN_MODES[mode],
                                 _ptr(wsb), wsb.numel(), _stream()))
    return h


def hgrn_scan_bwd(f, h, dh, h0=None, dh_last=None, mode: str = "auto", dx=None, df=None, want_dh0=False):
    """Derivative of the recurrence (mmf_hgrn_scan_bwd): f, h (the forward's output) and dh = dL/dh,
    all [b, t, d] fp32; returns (dx, df, dh0 or None)."""
    torch = _torch()
    lib = load()
    if f.shape != h.shape or f.shape != dh.shape or f.dim() != 3:
        raise ValueError("f, h and dh must all be [b, t, d]")
    for t_ in (f, h, dh):
        if t_.dtype != torch.float32 or not t_.is_contiguous():
            raise TypeError("f, h and dh must be contiguous float32")
    b, t, d = f.shape
    dx = dx if dx is not None else torch.empty_like(f)
    df = df if df is not None else torch.empty_like(f)
    dh0 = torch.empty((b, d), dtype=torch.float32, device=f.device) if want_dh0 else None
    _check(lib.mmf_hgrn_scan_bwd(_ptr(f), _ptr(h), _ptr(h0), _ptr(dh), _ptr(dh_last), _ptr(dx), _ptr(df),
                                 _ptr(dh0), b, t, d, SCAN_MODES[mode], _stream()))
    return dx, df, dh0


def hgrn2_scan_fwd(f, i, o, e: int, s0=None, out=None, s_last=None, mode: str = "auto"):
    """The expanded-state recurrence (mmf_hgrn2_scan_fwd) over f, i, o [b, t, d] fp32 with heads
    of e channels; s0 / s_last [b, d / e, e, e] fp32 or None (s_last may be s0); mode "auto",
    "recurrent" or "chunk". Returns y."""
    torch = _torch()
    lib = load()
    if f.shape != i.shape or f.shape != o.shape or f.dim() != 3:
        raise ValueError("f, i and o must all be [b, t, d]")
    for t_ in (f, i, o) + tuple(x for x in (s0, s_last) if x is not None):
        if t_.dtype != torch.float32 or not t_.is_contiguous():
            raise TypeError("f, i, o and the states must be contiguous float32")
    b, t, d = f.shape
    y = out if out is not None else torch.empty_like(f)
    _check(lib.mmf_hgrn2_scan_fwd(_ptr(f), _ptr(i), _ptr(o), _ptr(s0), _ptr(y), _ptr(s_last), b, t, d, e,
                                  SCAN_MODES[mode], _stream()))
    return y


@dataclass
class LayerParams:
    """Packed weights of one HGRNBit block."""
    i: PackedLinear
    f: PackedLinear
    g: PackedLinear
    o: PackedLinear
    gate: PackedLinear
    down: PackedLinear
    g_norm_w: Optional[object] = None
    eps: float = 1e-8

    @property
    def d(self) -> int:
        return self.i.k

    @property
    def inner(self) -> int:
        return self.down.k

    def c(self) -> CLayerWeights:
        return CLayerWeights(self.i.c(), self.f.c(), self.g.c(), self.o.c(), self.gate.c(), self.down.c(),
                             _ptr(self.g_norm_w), self.d, self.inner, self.eps)

    @classmethod
    def pack(cls, latent: dict, gains: Optional[dict] = None, eps: float = 1e-8) -> "LayerParams":
        """Pack latent device weights {i,f,g,o,gate,down} (+ optional device gains) with mmf_ternary_pack."""
        gains = gains or {}
        parts = {k: ternary_pack(latent[k], gains.get(k)) for k in ("i", "f", "g", "o", "gate", "down")}
        return cls(g_norm_w=gains.get("g_norm"), eps=eps, **parts)


class LayerProbe:
    """Device buffers receiving every stage of a layer call (validation only)."""

    def __init__(self, m: int, d: int, inner: int, device, shared_ifg: bool = True):
        torch = _torch()
        e = lambda *s, dt=torch.float32: torch.empty(s, dtype=dt, device=device)  # noqa: E731
        nq = 1 if shared_ifg else 3
        self.codes_x = [e(m, d, dt=torch.int8) for _ in range(nq)]
        self.scale_x = [e(m) for _ in range(nq)]
        self.acc_ifg = e(m, 3, d, dt=torch.int32)
        self.f, self.xt, self.g, self.h, self.u = (e(m, d) for _ in range(5))
        self.codes_u, self.scale_u, self.acc_o = e(m, d, dt=torch.int8), e(m), e(m, d, dt=torch.int32)
        self.x1 = e(m, d)
        self.codes_x1, self.scale_x1 = e(m, d, dt=torch.int8), e(m)
        self.acc_gate = e(m, 2 * inner, dt=torch.int32)
        self.z = e(m, inner)
        self.codes_z, self.scale_z = e(m, inner, dt=torch.int8), e(m)
        self.acc_down = e(m, d, dt=torch.int32)

    def c(self) -> CLayerProbe:
        p = CLayerProbe()
        for q in range(3):
            p.codes_x[q] = _ptr(self.codes_x[q]) if q < len(self.codes_x) else None
            p.scale_x[q] = _ptr(self.scale_x[q]) if q < len(self.scale_x) else None
        for name in PROBE_FIELDS:
            setattr(p, name, _ptr(getattr(self, name)))
        return p

    def host(self) -> dict:
        out = {}
        for name in ["codes_x", "scale_x"]:
            out[name] = [t.cpu().numpy() for t in getattr(self, name)]
        for name in PROBE_FIELDS:
            out[name] = getattr(self, name).cpu().numpy()
        return out


def layer_workspace_size(params: LayerParams, b: int, t: int) -> int:
    need = SZ(0)
    cw = params.c()
    _check(load().mmf_layer_workspace_size(ctypes.byref(cw), b, t, ctypes.byref(need)))
    return need.value


def layer_fwd(params: LayerParams, x, h0=None, want_h_last: bool = True, mode: str = "auto",
              probe: Optional[LayerProbe] = None, out=None, h_last=None, ws=None):
    """One HGRNBit block over x [b, t, d] (mmf_layer_fwd); returns (out, h_last)."""
    torch = _torch()
    lib = load()
    if x.dim() != 3 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [b, t, d] tensor")
    b, t, d = x.shape
    out = out if out is not None else torch.empty_like(x)
    if h_last is None and want_h_last:
        h_last = torch.empty((b, d), dtype=torch.float32, device=x.device)
    cw = params.c()
    need = SZ(0)
    _check(lib.mmf_layer_workspace_size(ctypes.byref(cw), b, t, ctypes.byref(need)))
    wsb = _workspace(need.value, x.device, ws)
    cp = probe.c() if probe is not None else None
    _check(lib.mmf_layer_fwd(ctypes.byref(cw), _ptr(x), _ptr(out), _dtype_code(x.dtype), b, t, _ptr(h0),
                             _ptr(h_last), SCAN_MODES[mode], _ptr(wsb), wsb.numel(),
                             ctypes.byref(cp) if cp is not None else None, _stream()))
    return out, h_last


LAYER_WEIGHTS = ("i", "f", "g", "o", "gate", "down")


def layer_bwd(params: LayerParams, x, dout, h0=None, dh_last=None, mode: str = "auto", want_dh0: bool = True,
              want_weights: bool = True, want_gains: bool = False, ws=None) -> dict:
    """Derivative of one block (mmf_layer_bwd, straight-through quantisers): x, dout [b, t, d];
    returns a dict with dx [b, t, d] fp32, dh0 [b, d], dw {name: [n, k]}, dgain {name: [k]} and
    dg_norm_w [d] (fp32; the parts not asked for are None)."""
    torch = _torch()
    lib = load()
    if x.dim() != 3 or not x.is_contiguous() or not dout.is_contiguous() or dout.shape != x.shape:
        raise ValueError("x and dout must be contiguous [b, t, d] tensors")
    b, t, d = x.shape
    dev = x.device
    lins = [getattr(params, n) for n in LAYER_WEIGHTS]
    res = dict(dx=torch.empty((b, t, d), dtype=torch.float32, device=dev),
               dh0=torch.empty((b, d), dtype=torch.float32, device=dev) if want_dh0 else None,
               dw={n: torch.empty((l.n, l.k), dtype=torch.float32, device=dev) for n, l in zip(LAYER_WEIGHTS, lins)}
               if want_weights else None,
               dgain={n: torch.empty((l.k,), dtype=torch.float32, device=dev) for n, l in zip(LAYER_WEIGHTS, lins)}
               if want_gains else None,
               dg_norm_w=torch.empty((d,), dtype=torch.float32, device=dev) if want_gains else None)
    cg = CLayerGrads()
    cg.dx = _ptr(res["dx"])
    cg.dh0 = _ptr(res["dh0"])
    for q, n in enumerate(LAYER_WEIGHTS):
        cg.dw[q] = _ptr(res["dw"][n]) if res["dw"] else None
        cg.dgain[q] = _ptr(res["dgain"][n]) if res["dgain"] else None
    cg.dg_norm_w = _ptr(res["dg_norm_w"])
    cw = params.c()
    need = SZ(0)
    _check(lib.mmf_layer_bwd_workspace_size(ctypes.byref(cw), b, t, ctypes.byref(need)))
    wsb = _workspace(need.value, dev, ws)
    _check(lib.mmf_layer_bwd(ctypes.byref(cw), _ptr(x), _ptr(dout), _dtype_code(x.dtype), b, t, _ptr(h0),
                             _ptr(dh_last), SCAN_MODES[mode], ctypes.byref(cg), _ptr(wsb), wsb.numel(), _stream()))
    return res


def layer_decode_step(params: LayerParams, x, h, probe: Optional[LayerProbe] = None, out=None, ws=None):
    """One token per sequence, x [b, d], state h [b, d] fp32 updated in place (mmf_layer_decode_step)."""
    torch = _torch()
    lib = load()
    if x.dim() != 2 or not x.is_contiguous() or not h.is_contiguous() or h.dtype != torch.float32:
        raise ValueError("x must be contiguous [b, d]; h contiguous float32 [b, d]")
    b, d = x.shape
    out = out if out is not None else torch.empty_like(x)
    cw = params.c()
    need = SZ(0)
    _check(lib.mmf_layer_workspace_size(ctypes.byref(cw), b, 1, ctypes.byref(need)))
    wsb = _workspace(need.value, x.device, ws)
    cp = probe.c() if probe is not None else None
    _check(lib.mmf_layer_decode_step(ctypes.byref(cw), _ptr(x), _ptr(out), _dtype_code(x.dtype), b, _ptr(h),
                                     _ptr(wsb), wsb.numel(), ctypes.byref(cp) if cp is not None else None,
                                     _stream()))
    return out


def layer_decode_step_noalloc(params: LayerParams, x, h, out, probe: Optional[LayerProbe] = None):
    """layer_decode_step with the library's own per-device scratch (mmf_layer_decode_step_noalloc):
    no workspace argument, nothing allocated by the call; `out` [b, d] must be given."""
    torch = _torch()
    if x.dim() != 2 or not x.is_contiguous() or not h.is_contiguous() or h.dtype != torch.float32:
        raise ValueError("x must be contiguous [b, d]; h contiguous float32 [b, d]")
    if out is None or out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like x")
    b = x.shape[0]
    cw = params.c()
    cp = probe.c() if probe is not None else None
    _check(load().mmf_layer_decode_step_noalloc(ctypes.byref(cw), _ptr(x), _ptr(out), _dtype_code(x.dtype), b,
                                                _ptr(h), ctypes.byref(cp) if cp is not None else None, _stream()))
    return out


class StackDecoder:
    """A stack of blocks and their states bound to one workspace (mmf_stack_decode_bind, which
    synchronises once); step(x) runs one token per sequence through every block in one
    persistent kernel (mmf_stack_decode_step) and updates the states in place."""

    def __init__(self, layers: list, states: list, b: int, ws=None):
        torch = _torch()
        lib = load()
        if len(layers) != len(states) or not layers:
            raise ValueError("one state per block, at least one block")
        for h in states:
            if h.dtype != torch.float32 or not h.is_contiguous() or tuple(h.shape) != (b, layers[0].d):
                raise ValueError("each state must be a contiguous float32 [b, d] tensor")
        self.layers, self.states, self.b = list(layers), list(states), b
        self._cw = (CLayerWeights * len(layers))(*[p.c() for p in layers])
        need = SZ(0)
        _check(lib.mmf_stack_decode_workspace_size(self._cw, len(layers), b, ctypes.byref(need)))
        self.ws = _workspace(need.value, states[0].device, ws)
        hp = (P * len(states))(*[_ptr(h) for h in states])
        _check(lib.mmf_stack_decode_bind(self._cw, len(layers), b, hp, _ptr(self.ws), self.ws.numel(), _stream()))

    def step(self, x, out=None):
        torch = _torch()
        if x.dim() != 2 or not x.is_contiguous() or x.shape[0] != self.b:
            raise ValueError("x must be a contiguous [b, d] tensor")
        out = out if out is not None else torch.empty_like(x)
        _check(load().mmf_stack_decode_step(self._cw, len(self.layers), _ptr(x), _ptr(out), _dtype_code(x.dtype),
                                            self.b, _ptr(self.ws), self.ws.numel(), _stream()))
        return out


def stack_decode_expired() -> int:
    """Barrier waits of the stack decode kernel that expired since the library was loaded (synchronous)."""
    c = ctypes.c_uint32(0)
    _check(load().mmf_stack_decode_expired(ctypes.byref(c)))
    return c.value
