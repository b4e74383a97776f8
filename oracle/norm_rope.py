"""Plain CPU oracle for the fused RMSNorm + RoPE step.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the benchmark's
CPU-baseline leg; never by the product path.  It shares no code, table or
constant with the HIP library.

Source: the "Ultra LLM Engine" page lists, among its fused kernels, RMSNorm
followed by RoPE (Core Components > Fused Kernels, third bullet; the
Architecture diagram puts "RMSNorm + RoPE" first in each QuantizedTransformer
layer, ahead of the quantized Q/K/V/O projections).  The page names the two
steps and fixes none of their arithmetic, so each step below is a reading:

  R-RN  RMSNorm over the last dimension D of each vector (one attention head
        of D = head_dim, or a whole hidden vector with one "head"):
            u = x / sqrt(mean(x^2) + eps) * gamma
        with a learned per-dimension gain gamma [D] and a caller-given eps.
  R-RP  RoPE in the rotate-half pairing: element i pairs with element i + D/2
        (i < D/2); pair i turns by the angle p * theta^(-2i/D), p being the
        vector's token position:  (a, b) -> (a cos - b sin, b cos + a sin).
  R-RT  The angles enter through a table of cos and sin, [max_pos, D/2] fp32,
        built once: each entry is the fp32 rounding (to nearest even) of the
        cosine / sine of the angle formed exactly (fp64).  Kernel and oracle
        read the same table; the table builder is checked against closed forms.
  R-RO  x and y are fp16, gamma fp32; the reference below is exact (fp64).  A
        kernel computing in fp32 and rounding to fp16 once must land within
        one fp16 spacing of it, plus the fp32 rounding of the vector's scale
        (2^-18 of its largest value) where cancellation makes a value tiny.
"""
from __future__ import annotations

import numpy as np

__all__ = ["rope_table", "rmsnorm_rope", "fp16_spacing", "within_gate"]


def rope_table(theta: float, d: int, max_pos: int):
    """(cos, sin), each fp32 [max_pos, d/2]: angle(p, i) = p * theta**(-2i/d) (R-RP, R-RT)."""
    if d % 2:
        raise ValueError("head dimension must be even")
    i = np.arange(d // 2, dtype=np.float64)
    inv_freq = np.float64(theta) ** (-2.0 * i / d)
    angle = np.arange(max_pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(angle).astype(np.float32), np.sin(angle).astype(np.float32)


def rmsnorm_rope(x16: np.ndarray, gamma: np.ndarray, pos: np.ndarray, cos: np.ndarray,
                 sin: np.ndarray, eps) -> np.ndarray:
    """y [T, H, D] in fp64 from x fp16 [T, H, D], gamma fp32 [D], pos int [T] (R-RN, R-RP).

    Step 1, RMSNorm: u = x * (mean over D of x^2 + eps)^(-1/2) * gamma.
    Step 2, RoPE: with h = D/2, c = cos[pos], s = sin[pos]:
        y[:h] = u[:h] * c - u[h:] * s,   y[h:] = u[h:] * c + u[:h] * s.
    """
    x = np.asarray(x16).astype(np.float64)
    d = x.shape[-1]
    h = d // 2
    eps64 = np.float64(np.float32(eps))
    ms = np.mean(x * x, axis=-1, keepdims=True)
    u = x / np.sqrt(ms + eps64) * np.asarray(gamma, dtype=np.float32).astype(np.float64)
    c = np.asarray(cos, dtype=np.float32)[np.asarray(pos)].astype(np.float64)[:, None, :]
    s = np.asarray(sin, dtype=np.float32)[np.asarray(pos)].astype(np.float64)[:, None, :]
    a, b = u[..., :h], u[..., h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def within_gate(y: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """R-RO gate: |y - ref| <= one fp16 spacing at |ref| + 2^-18 * max |ref| of the vector.

    The second term is the fp32 arithmetic on values of the vector's scale
    (a few roundings of 2^-24 each, with headroom), which dominates only where
    a rotated value lands near zero by cancellation."""
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.abs(ref).max(axis=-1, keepdims=True)
    return np.abs(np.asarray(y, dtype=np.float64) - ref) <= fp16_spacing(ref) + 2.0 ** -18 * scale


def fp16_spacing(y: np.ndarray) -> np.ndarray:
    """Distance between adjacent fp16 values at |y| (2^-24 in the subnormal range)."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return np.exp2(e - 10)
