"""Seeded synthetic inputs shared by the oracle-side and the GPU-side tests.

This module only draws random numbers (numpy PCG64) and rounds them to the
input dtype; it contains none of the layer's arithmetic, so both sides can
consume the same host tensors.

Recipes follow the workloads of the MatMul-free LM models (model sizes from
"MatMul-Free LM：把矩陣乘法從語言模型裡拿掉之後，剩下什麼", section
"三個預訓練模型的實際差異"; MLP widths from section "HGRNBitBlock 的結構"):
activations x ~ N(0, 1), latent weights ~ N(0, 0.02) (ternarised by each side
on its own), RMSNorm gains 1 unless a test asks for N(1, 0.1) gains.
"""
from __future__ import annotations

import numpy as np

# hidden size d, MLP inner size, layer count
SHAPES = {
    "370M": (1024, 2816, 24),
    "1.3B": (2048, 5632, 24),
    "2.7B": (2560, 6912, 32),
}

PROJECTIONS = ("i", "f", "g", "o", "gate", "down")


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returned as float32."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    bits = a.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    out = rounded.astype(np.uint32).view(np.float32)
    return np.where(np.isnan(a), a, out).astype(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are exactly bfloat16."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def activations(shape, seed: int, dtype: str = "f32", std: float = 1.0) -> np.ndarray:
    """x ~ N(0, std^2) as float32 (values exactly representable in ``dtype``)."""
    x = (rng(seed).standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)
    return bf16_round(x) if dtype == "bf16" else x


def latent_weights(d: int, inner: int, seed: int, std: float = 0.02) -> dict:
    """Latent fp32 weights of one block: i/f/g/o [d,d], gate [2*inner, d], down [d, inner]."""
    g = rng(seed)
    shapes = {"i": (d, d), "f": (d, d), "g": (d, d), "o": (d, d),
              "gate": (2 * inner, d), "down": (d, inner)}
    return {k: (g.standard_normal(size=shapes[k], dtype=np.float32) * np.float32(std)).astype(np.float32)
            for k in PROJECTIONS}


def norm_gains(d: int, inner: int, seed: int, std: float = 0.1) -> dict:
    """RMSNorm gains ~ N(1, std^2) for every projection and for g_norm."""
    g = rng(seed)
    sizes = {"i": d, "f": d, "g": d, "o": d, "gate": d, "down": inner, "g_norm": d}
    return {k: (1.0 + std * g.standard_normal(size=n)).astype(np.float32) for k, n in sizes.items()}


def scan_inputs(b: int, t: int, d: int, seed: int, f_loc: float = 2.0, f_scale: float = 1.0):
    """Scan-only inputs: x ~ N(0,1); f drawn from a logit-normal (logit ~ N(f_loc, f_scale^2))."""
    g = rng(seed)
    x = g.standard_normal(size=(b, t, d), dtype=np.float32)
    logit = g.standard_normal(size=(b, t, d), dtype=np.float32) * np.float32(f_scale) + np.float32(f_loc)
    f = (1.0 / (1.0 + np.exp(-logit.astype(np.float64)))).astype(np.float32)
    return x, f


def hgrn2_inputs(b: int, t: int, d: int, seed: int, f_loc: float = 2.0, f_scale: float = 1.0):
    """Inputs of the expanded-state recurrence: f as in ``scan_inputs`` (logit-normal), the input
    vector i and the output gate o ~ N(0, 1); all fp32 [b, t, d]."""
    g = rng(seed)
    logit = g.standard_normal(size=(b, t, d), dtype=np.float32) * np.float32(f_scale) + np.float32(f_loc)
    f = (1.0 / (1.0 + np.exp(-logit.astype(np.float64)))).astype(np.float32)
    i = g.standard_normal(size=(b, t, d), dtype=np.float32)
    o = g.standard_normal(size=(b, t, d), dtype=np.float32)
    return f, i, o


def layer_seed(config_seed: int, layer: int) -> int:
    return config_seed * 1000 + layer
