"""CPU oracle for the HGRNBit layer forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package. The product path (the HIP
library and its binding) never does; the two share no code.

What it computes, and where each step comes from (web pages about the
MatMul-free LM project):

* [R1] "MatMul-Free LLM 深度分析报告" (nightvoyager.top), section "核心价值提炼":
  table "创新之处" -- ternary ``weight_quant`` (round to nearest {-1,0,+1}),
  the HGRN recurrence h_t = gate_t * h_{t-1} + x_t (elementwise); list
  "可复用的模式与技巧" -- RMSNorm fused with INT8 activation quantisation,
  RMSNorm fused with a Swish gate.
* [R3] "MatMul-Free LM：把矩陣乘法從語言模型裡拿掉之後，剩下什麼" (hysenlabs.com),
  section "HGRNBitBlock 的結構": a block is a token mixer with four
  FusedBitLinear projections i/f/g/o (each with an eps = 1e-8 RMSNorm) and a
  g_norm RMSNorm-Swish gate, followed by an MLP of gate_proj (2x inner
  outputs), a SiLU and down_proj.
* [R4] mooersco.com article, section 4.1: a ternary matrix-vector product is a
  conditional add / subtract per weight.

Where the pages are silent the stated problem fixes the reading: per-token
absmax int8 scale (127 / amax), per-tensor mean-|W| weight scale, forget gate
f = sigmoid(f_proj), input x~ = (1 - f) * SiLU(i_proj), SiLU-gated MLP over the
two halves of gate_proj. Further readings (the 1e-5 floors, round half to
even, g_norm's eps, the residual wiring, which half of gate_proj is gated)
are listed in the project's design notes.

Beyond the forward pass, for training through the quantisers with a
straight-through estimator ([R1] list "可复用的模式与技巧"): ``hgrn_scan_bwd``,
the derivative of the recurrence (reverse time), and ``bitlinear_bwd``, the
derivative of FusedBitLinear with both quantisers passed straight through;
and for the token-to-token loop of generation, ``embed`` and ``greedy_head``
(a FusedBitLinear head whose largest exact sum picks the next token).
``hgrn2_scan`` widens the recurrence's state from a vector to a matrix per head
(HGRN2, which [R1] names without printing its equations: a reading, stated
in its docstring).

Precision: every step is binary64 except the two quantisers, which decide
integers and therefore run in the kernel's precision (binary32 operations,
binary64 sum of squares); their input vector is rounded to binary32 first.
The ternary contraction is exact integer arithmetic.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MMF_ORACLE_LIB: another build of the same C source (the sanitizer check loads one)
_LIB_PATH = os.environ.get("MMF_ORACLE_LIB") or os.path.join(_HERE, "libmmf_oracle.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_quant_rows.argtypes = [P, I64, I64, P, ctypes.c_float, P, P, P]
    lib.oracle_ternarize.argtypes = [P, I64, I64, P, P]
    lib.oracle_pack.argtypes = [P, I64, I64, P]
    lib.oracle_unpack.argtypes = [P, I64, I64, P]
    lib.oracle_ternary_matmul.argtypes = [P, P, I64, I64, I64, P]
    lib.oracle_hgrn_scan.argtypes = [P, P, P, I64, I64, I64, P]
    lib.oracle_hgrn_scan_bwd.argtypes = [P, P, P, P, P, I64, I64, I64, P, P, P]
    for fn in (lib.oracle_quant_rows, lib.oracle_ternarize, lib.oracle_pack, lib.oracle_unpack,
               lib.oracle_ternary_matmul, lib.oracle_hgrn_scan, lib.oracle_hgrn_scan_bwd, lib.oracle_num_threads):
        fn.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


# ---------------------------------------------------------------------------
# Quantisers (binary32 decisions)
# ---------------------------------------------------------------------------

def quantize(v: np.ndarray, gain: Optional[np.ndarray] = None, eps: float = 1e-8):
    """RMSNorm (eps inside the square root) + per-row absmax int8 codes.

    [R1] fused RMSNorm + INT8 quantisation; [R3] eps = 1e-8. ``v`` is rounded
    to binary32 first (the kernel's precision). Returns (q int8 [m,k],
    s float32 [m], sumq int32 [m]) with q ~= RMSNorm(v)*gain*s.
    """
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
    k = v.shape[-1]
    m = v.size // k
    g = None if gain is None else np.ascontiguousarray(np.asarray(gain, dtype=np.float32))
    if g is not None and g.shape != (k,):
        raise ValueError("gain must have shape (k,)")
    q = np.empty(v.shape, dtype=np.int8)
    s = np.empty(v.shape[:-1], dtype=np.float32)
    sq = np.empty(v.shape[:-1], dtype=np.int32)
    rc = _load().oracle_quant_rows(_ptr(v), m, k, _ptr(g), ctypes.c_float(eps), _ptr(q), _ptr(s), _ptr(sq))
    if rc != 0:
        raise ValueError("oracle_quant_rows failed")
    return q, s, sq


def ternarize(w: np.ndarray):
    """Round-to-nearest ternary codes with a per-tensor mean-|W| scale ([R1] weight_quant).

    Returns (t int8 [n,k] in {-1,0,1}, mu float32).
    """
    w = np.ascontiguousarray(np.asarray(w, dtype=np.float32))
    n, k = w.shape
    t = np.empty((n, k), dtype=np.int8)
    mu = np.zeros(1, dtype=np.float32)
    if _load().oracle_ternarize(_ptr(w), n, k, _ptr(t), _ptr(mu)) != 0:
        raise ValueError("oracle_ternarize failed")
    return t, np.float32(mu[0])


def weight_scale(mu) -> np.float32:
    """sw = 1 / max(mu, 1e-5) in binary32: ternary t approximates W * sw."""
    return np.float32(np.float32(1.0) / np.maximum(np.float32(mu), np.float32(1e-5)))


def pack(t: np.ndarray) -> np.ndarray:
    """2-bit packing of codes c = t + 1, 16 per uint32 word ([R4] section 5.1)."""
    t = np.ascontiguousarray(np.asarray(t, dtype=np.int8))
    n, k = t.shape
    if k % 16:
        raise ValueError("k must be a multiple of 16")
    words = np.empty((n, k // 16), dtype=np.uint32)
    if _load().oracle_pack(_ptr(t), n, k, _ptr(words)) != 0:
        raise ValueError("oracle_pack failed (k % 16 or a code outside {-1,0,1})")
    return words


def unpack(words: np.ndarray, k: int) -> np.ndarray:
    words = np.ascontiguousarray(np.asarray(words, dtype=np.uint32))
    n = words.shape[0]
    t = np.empty((n, k), dtype=np.int8)
    if _load().oracle_unpack(_ptr(words), n, k, _ptr(t)) != 0:
        raise ValueError("oracle_unpack failed")
    return t


def ternary_matmul(q: np.ndarray, t: np.ndarray) -> np.ndarray:
    """Exact acc[i, o] = sum_k q[i, k] * t[o, k] ([R4] section 4.1), int32."""
    q = np.ascontiguousarray(np.asarray(q, dtype=np.int8))
    t = np.ascontiguousarray(np.asarray(t, dtype=np.int8))
    k = q.shape[-1]
    m = q.size // k
    n = t.shape[0]
    if t.shape[1] != k:
        raise ValueError("inner dimensions differ")
    acc = np.empty(q.shape[:-1] + (n,), dtype=np.int32)
    rc = _load().oracle_ternary_matmul(_ptr(q), _ptr(t), m, n, k, _ptr(acc))
    if rc != 0:
        raise ValueError("oracle_ternary_matmul failed (%d)" % rc)
    return acc


def dequant(acc: np.ndarray, s: np.ndarray, mu) -> np.ndarray:
    """acc / (s * sw) in binary64: the float contraction of the dequantised operands."""
    sw = np.float64(weight_scale(mu))
    return np.asarray(acc, dtype=np.float64) / (np.asarray(s, dtype=np.float64)[..., None] * sw)


# ---------------------------------------------------------------------------
# binary64 elementwise pieces
# ---------------------------------------------------------------------------

def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z * sigmoid(z)


def bitlinear(x: np.ndarray, t: np.ndarray, mu, gain=None, eps: float = 1e-8):
    """FusedBitLinear: RMSNorm + int8 quant of x, exact ternary contraction, dequant; no bias."""
    q, s, sq = quantize(x, gain, eps)
    acc = ternary_matmul(q, t)
    return dict(y=dequant(acc, s, mu), q=q, s=s, sumq=sq, acc=acc)


def bitlinear_bwd(x: np.ndarray, t: np.ndarray, mu, dy: np.ndarray, gain=None, eps: float = 1e-8):
    """Derivative of ``bitlinear`` with straight-through quantisers, binary64.

    [R1] list "可复用的模式与技巧": ``weight_quant`` quantises in the forward pass and lets
    the gradient through unchanged in the backward pass (straight-through estimator); the
    same reading is taken for the activation quantiser. With u = RMSNorm(x) * gain, the
    dequantised operands u^ = q / s and W^ = t / sw of the forward product y = u^ W^T:
        du = dy W^                     (the activation quantiser passes du to u)
        dW = dy^T u^                   (weight_quant passes dW^ to the latent W)
        r = (mean(x^2) + eps)^(-1/2),  c = sum_k x_k gain_k du_k
        dx_k = r gain_k du_k - (r^3 / K) x_k c,   dgain_k = sum_rows du_k x_k r
    Returns (dx [m,k], dW [n,k], dgain [k]).
    """
    x64 = np.asarray(x, dtype=np.float64)
    dy64 = np.asarray(dy, dtype=np.float64)
    k = x64.shape[-1]
    q, s, _ = quantize(x, gain, eps)
    sw = np.float64(weight_scale(mu))
    w_hat = np.asarray(t, dtype=np.float64) / sw
    u_hat = q.astype(np.float64) / s.astype(np.float64)[:, None]
    du = dy64 @ w_hat
    dw = dy64.T @ u_hat
    g = np.ones(k) if gain is None else np.asarray(gain, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x64 * x64, axis=1) + np.float64(np.float32(eps)))
    c = np.sum(x64 * g * du, axis=1)
    dx = r[:, None] * g * du - (r ** 3 / k)[:, None] * x64 * c[:, None]
    dgain = np.sum(du * x64 * r[:, None], axis=0)
    return dx, dw, dgain


def embed(ids: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Rows of an embedding table for token ids; an id outside [0, vocab) gives a zero row
    (the token-to-token loop of generation; [R3] section "安裝與初始化：三行指令與一個 config
    物件": the default config has 32000 tokens, width 2048, 24 layers, and a generation example)."""
    ids = np.asarray(ids, dtype=np.int64)
    table = np.asarray(table)
    out = np.zeros((ids.size, table.shape[1]), dtype=table.dtype)
    ok = (ids >= 0) & (ids < table.shape[0])
    out[ok] = table[ids[ok]]
    return out


def first_argmax(acc: np.ndarray) -> np.ndarray:
    """Per row, the smallest index holding the row's largest value (a plain scan)."""
    acc = np.asarray(acc)
    out = np.empty(acc.shape[0], dtype=np.int32)
    for r in range(acc.shape[0]):
        best, arg = acc[r, 0], 0
        for j in range(1, acc.shape[1]):
            if acc[r, j] > best:
                best, arg = acc[r, j], j
        out[r] = arg
    return out


def greedy_head(x: np.ndarray, t: np.ndarray, mu, gain=None, eps: float = 1e-8) -> dict:
    """Greedy next token from a FusedBitLinear head: the head's logits are acc * dq with one
    dq > 0 per row, so the largest logit is the largest exact int32 sum acc; ties go to the
    smallest token id. Returns the head's bitlinear result plus ``tokens`` [m] int32."""
    r = bitlinear(x, t, mu, gain, eps)
    r["tokens"] = first_argmax(r["acc"])
    return r


def mixer_gates(i_hat, f_hat):
    """f = sigmoid(f_proj); x~ = (1 - f) * SiLU(i_proj)."""
    f = sigmoid(f_hat)
    return f, (1.0 - f) * silu(i_hat)


def hgrn_scan(x: np.ndarray, f: np.ndarray, h0: Optional[np.ndarray] = None) -> np.ndarray:
    """h_t = f_t * h_{t-1} + x_t per (batch, channel), binary64, sequential ([R1])."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    f = np.ascontiguousarray(np.asarray(f, dtype=np.float64))
    if x.shape != f.shape or x.ndim != 3:
        raise ValueError("x and f must both be [b, t, d]")
    b, t, d = x.shape
    h0a = None if h0 is None else np.ascontiguousarray(np.asarray(h0, dtype=np.float64).reshape(b, d))
    h = np.empty_like(x)
    if _load().oracle_hgrn_scan(_ptr(x), _ptr(f), _ptr(h0a), b, t, d, _ptr(h)) != 0:
        raise ValueError("oracle_hgrn_scan failed")
    return h


def hgrn_scan_bwd(f: np.ndarray, h: np.ndarray, dh: np.ndarray, h0: Optional[np.ndarray] = None,
                  dh_last: Optional[np.ndarray] = None):
    """Derivative of ``hgrn_scan`` for a loss with dL/dh = dh and dL/dh_last = dh_last, binary64,
    sequential from the last step: D_t = dh_t + f_{t+1} D_{t+1} (D_{T-1} = dh_{T-1} + dh_last);
    returns dx = D, df = D * h_{t-1} (h_{-1} = h0 or 0) and dh0 = f_0 D_0 (the recurrence of [R1]
    table "创新之处", differentiated)."""
    f = np.ascontiguousarray(np.asarray(f, dtype=np.float64))
    h = np.ascontiguousarray(np.asarray(h, dtype=np.float64))
    dh = np.ascontiguousarray(np.asarray(dh, dtype=np.float64))
    if f.shape != h.shape or f.shape != dh.shape or f.ndim != 3:
        raise ValueError("f, h and dh must all be [b, t, d]")
    b, t, d = f.shape
    h0a = None if h0 is None else np.ascontiguousarray(np.asarray(h0, dtype=np.float64).reshape(b, d))
    gla = None if dh_last is None else np.ascontiguousarray(np.asarray(dh_last, dtype=np.float64).reshape(b, d))
    dx = np.empty_like(f)
    df = np.empty_like(f)
    dh0 = np.empty((b, d), dtype=np.float64)
    if _load().oracle_hgrn_scan_bwd(_ptr(f), _ptr(h), _ptr(h0a), _ptr(dh), _ptr(gla), b, t, d, _ptr(dx), _ptr(df),
                                    _ptr(dh0)) != 0:
        raise ValueError("oracle_hgrn_scan_bwd failed")
    return dx, df, dh0


def hgrn2_scan(f: np.ndarray, i: np.ndarray, o: np.ndarray, e: int, s0: Optional[np.ndarray] = None):
    """The HGRN recurrence with an expanded state (HGRN2), binary64, sequential.

    [R1] names HGRN2 as the gated linear recurrence that replaces attention (section
    "核心价值提炼", table "创新之处" and list "关键设计决策") and prints only its elementwise form
    h_t = g_t * h_{t-1} + x_t. The expanded state is a reading: the channels split into heads of e,
    each head's state is an e x e matrix, the forget gate acts on its rows, the input is the outer
    product of (1 - f) with the input vector and the output gate reads the state out:

        S_t[a][c] = f_t[a] * S_{t-1}[a][c] + (1 - f_t[a]) * i_t[c]
        y_t[c]    = sum_a o_t[a] * S_t[a][c]

    (a, c index the head's e channels). With e = 1 this is [R1]'s recurrence with
    x~ = (1 - f) * i, read out as y = o * h.
    f, i, o: [b, t, d] with d a multiple of e; s0: [b, d / e, e, e] or None (zeros).
    Returns (y [b, t, d], s_last [b, d / e, e, e])."""
    f = np.asarray(f, dtype=np.float64)
    i = np.asarray(i, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    if f.shape != i.shape or f.shape != o.shape or f.ndim != 3:
        raise ValueError("f, i and o must all be [b, t, d]")
    b, t, d = f.shape
    if e < 1 or d % e:
        raise ValueError("d must be a multiple of e")
    nh = d // e
    fh = f.reshape(b, t, nh, e)
    ih = i.reshape(b, t, nh, e)
    oh = o.reshape(b, t, nh, e)
    s = np.zeros((b, nh, e, e)) if s0 is None else np.array(s0, dtype=np.float64).reshape(b, nh, e, e)
    y = np.empty((b, t, nh, e))
    for step in range(t):
        fa = fh[:, step][..., :, None]                  # forget gate on the rows
        s = fa * s + (1.0 - fa) * ih[:, step][..., None, :]
        y[:, step] = np.einsum("bna,bnac->bnc", oh[:, step], s)
    return y.reshape(b, t, d), s


def gnorm_swish(h, g, weight=None, eps: float = 1e-8):
    """g_norm: RMSNorm(h) * weight, gated by Swish(g) ([R1] RMSNorm + Swish gate)."""
    h = np.asarray(h, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + np.float64(np.float32(eps)))
    u = h * r
    if weight is not None:
        u = u * np.asarray(weight, dtype=np.float64)
    return u * silu(g)


# ---------------------------------------------------------------------------
# Layer
# ---------------------------------------------------------------------------

@dataclass
class TernaryLinear:
    """One FusedBitLinear: ternary codes t [n,k], their scale mu, the RMSNorm gain."""
    t: np.ndarray
    mu: np.float32
    gain: Optional[np.ndarray] = None

    @classmethod
    def from_latent(cls, w: np.ndarray, gain: Optional[np.ndarray] = None) -> "TernaryLinear":
        t, mu = ternarize(w)
        return cls(t=t, mu=mu, gain=None if gain is None else np.asarray(gain, np.float32))

    def __call__(self, v, eps):
        return bitlinear(v, self.t, self.mu, self.gain, eps)


@dataclass
class Layer:
    """HGRNBit block weights ([R3] section "HGRNBitBlock 的結構")."""
    i: TernaryLinear
    f: TernaryLinear
    g: TernaryLinear
    o: TernaryLinear
    gate: TernaryLinear          # [2*inner, d]; rows [0, inner) are the SiLU branch
    down: TernaryLinear          # [d, inner]
    g_norm_w: Optional[np.ndarray] = None
    eps: float = 1e-8

    @property
    def d(self) -> int:
        return self.i.t.shape[1]

    @property
    def inner(self) -> int:
        return self.down.t.shape[1]


def layer_forward(L: Layer, x: np.ndarray, h0: Optional[np.ndarray] = None) -> dict:
    """HGRNBit block over a [b, t, d] sequence.

    Token mixer: i/f/g FusedBitLinear of x, gates, HGRN recurrence along t,
    g_norm, o_proj; residual x1 = x + o. MLP: gate_proj of x1, SiLU(first
    half) * second half, down_proj; out = x1 + mlp. No extra block-level norm:
    each FusedBitLinear normalises its own input. Returns every stage.
    """
    x = np.asarray(x, dtype=np.float64)
    b, t, d = x.shape
    eps = L.eps
    ri, rf, rg = L.i(x, eps), L.f(x, eps), L.g(x, eps)
    f, xt = mixer_gates(ri["y"], rf["y"])
    h = hgrn_scan(xt, f, h0)
    u = gnorm_swish(h, rg["y"], L.g_norm_w, eps)
    ro = L.o(u, eps)
    x1 = x + ro["y"]
    rgate = L.gate(x1, eps)
    inner = L.inner
    a, bb = rgate["y"][..., :inner], rgate["y"][..., inner:]
    z = silu(a) * bb
    rd = L.down(z, eps)
    out = x1 + rd["y"]
    return dict(out=out, h=h, h_last=h[:, -1, :] if t > 0 else None, f=f, xt=xt,
                i_hat=ri["y"], f_hat=rf["y"], g_hat=rg["y"], u=u, x1=x1, z=z,
                q_i=ri["q"], s_i=ri["s"], q_f=rf["q"], s_f=rf["s"], q_g=rg["q"], s_g=rg["s"],
                acc_i=ri["acc"], acc_f=rf["acc"], acc_g=rg["acc"],
                q_u=ro["q"], s_u=ro["s"], acc_o=ro["acc"],
                q_x1=rgate["q"], s_x1=rgate["s"], acc_gate=rgate["acc"],
                q_z=rd["q"], s_z=rd["s"], acc_down=rd["acc"])


def layer_decode_step(L: Layer, x: np.ndarray, h: np.ndarray) -> dict:
    """One token per sequence ([b, d]) with the carried state h [b, d]."""
    r = layer_forward(L, np.asarray(x, np.float64)[:, None, :], h0=h)
    return dict(out=r["out"][:, 0, :], h=r["h_last"], stages=r)


def dsilu(z):
    """d SiLU(z) / dz = sigmoid(z) (1 + z (1 - sigmoid(z)))."""
    z = np.asarray(z, dtype=np.float64)
    sg = sigmoid(z)
    return sg * (1.0 + z * (1.0 - sg))


def layer_backward(L: Layer, x: np.ndarray, dout: np.ndarray, h0: Optional[np.ndarray] = None,
                   dh_last: Optional[np.ndarray] = None, stages: Optional[dict] = None) -> dict:
    """Derivative of ``layer_forward`` with straight-through quantisers, binary64, for a loss
    with dL/dout = dout and dL/dh_last = dh_last. Every FusedBitLinear goes through
    ``bitlinear_bwd``; the rest is the chain rule through the block, last step first:
    MLP (SiLU product), o_proj, g_norm (RMSNorm of h times weight times SiLU(g)), the
    recurrence (``hgrn_scan_bwd``), the gates f = sigmoid(f^), x~ = (1 - f) SiLU(i^), and the
    i/f/g projections, whose input derivatives add to the residual path's. Returns dx, dh0,
    the latent weights' derivatives ``dw``, the gains' ``dgain`` (derivative at 1 where a
    projection has no gain), ``dg_norm_w`` and the intermediate derivatives.

    ``stages`` (optional) supplies the forward values the chain is evaluated at -- i_hat, f, g
    (as g_norm saw it), h, u, x1, ab (= [a | b]) and z, each [b*t, ...] -- in place of the
    oracle's own forward, so that a derivative can be checked at another implementation's
    forward values (its quantisers then see the same inputs)."""
    x = np.asarray(x, dtype=np.float64)
    b, t, d = x.shape
    m, inner, eps = b * t, L.inner, L.eps
    if stages is None:
        r = layer_forward(L, x, h0)
        st = dict(i_hat=r["i_hat"], f=r["f"], g=r["g_hat"], h=r["h"], u=r["u"], x1=r["x1"], z=r["z"])
        st["ab"] = L.gate(np.asarray(r["x1"]).reshape(m, d), eps)["y"]
    else:
        st = stages
    st = {k: np.asarray(v, dtype=np.float64).reshape(m, -1) for k, v in st.items()}
    dO = np.asarray(dout, dtype=np.float64).reshape(m, d)
    # MLP: out = x1 + down(z), z = SiLU(a) * b with [a | b] = gate(x1)
    x1, z, ab = st["x1"], st["z"], st["ab"]
    dz, dw_down, dg_down = bitlinear_bwd(z, L.down.t, L.down.mu, dO, L.down.gain, eps)
    a, bb = ab[:, :inner], ab[:, inner:]
    da = dz * bb * dsilu(a)
    db = dz * silu(a)
    dx1_gate, dw_gate, dg_gate = bitlinear_bwd(x1, L.gate.t, L.gate.mu, np.concatenate([da, db], axis=1),
                                               L.gate.gain, eps)
    dx1 = dO + dx1_gate
    # o_proj: x1 = x + o(u)
    u = st["u"]
    du, dw_o, dg_o = bitlinear_bwd(u, L.o.t, L.o.mu, dx1, L.o.gain, eps)
    # g_norm: u = (h r_h) * w * SiLU(g^)
    h = st["h"]
    gh = st["g"]
    rh = 1.0 / np.sqrt(np.mean(h * h, axis=1) + np.float64(np.float32(eps)))
    nrm = h * rh[:, None]
    w = np.ones(d) if L.g_norm_w is None else np.asarray(L.g_norm_w, dtype=np.float64)
    sg = silu(gh)
    dn = du * w * sg
    dg_norm_w = np.sum(du * nrm * sg, axis=0)
    dg_hat = du * nrm * w * dsilu(gh)
    c = np.sum(h * dn, axis=1)
    dh = rh[:, None] * dn - (rh ** 3 / d)[:, None] * h * c[:, None]
    # the recurrence, then the gates
    f, ih = st["f"], st["i_hat"]
    dxt, df, dh0 = hgrn_scan_bwd(f.reshape(b, t, d), h.reshape(b, t, d), dh.reshape(b, t, d), h0, dh_last)
    dxt, df = dxt.reshape(m, d), df.reshape(m, d)
    df_hat = (df - dxt * silu(ih)) * f * (1.0 - f)
    di_hat = dxt * (1.0 - f) * dsilu(ih)
    # i/f/g projections of x, plus the residual path
    X = x.reshape(m, d)
    dx_i, dw_i, dg_i = bitlinear_bwd(X, L.i.t, L.i.mu, di_hat, L.i.gain, eps)
    dx_f, dw_f, dg_f = bitlinear_bwd(X, L.f.t, L.f.mu, df_hat, L.f.gain, eps)
    dx_g, dw_g, dg_g = bitlinear_bwd(X, L.g.t, L.g.mu, dg_hat, L.g.gain, eps)
    dx = dx1 + dx_i + dx_f + dx_g
    return dict(dx=dx.reshape(b, t, d), dh0=dh0,
                dw=dict(i=dw_i, f=dw_f, g=dw_g, o=dw_o, gate=dw_gate, down=dw_down),
                dgain=dict(i=dg_i, f=dg_f, g=dg_g, o=dg_o, gate=dg_gate, down=dg_down),
                dg_norm_w=dg_norm_w, dz=dz, da=da, db=db, dx1=dx1, du=du, dh=dh, dxt=dxt, df=df,
                di_hat=di_hat, df_hat=df_hat, dg_hat=dg_hat)


def make_layer(latent: dict, gains: Optional[dict] = None, eps: float = 1e-8) -> Layer:
    """Ternarise a dict of latent fp32 weights {i,f,g,o,gate,down} (+ optional gains)."""
    gains = gains or {}
    parts = {k: TernaryLinear.from_latent(latent[k], gains.get(k)) for k in ("i", "f", "g", "o", "gate", "down")}
    return Layer(g_norm_w=gains.get("g_norm"), eps=eps, **parts)
