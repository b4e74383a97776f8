"""Plain CPU oracle for dynamic activation quantization and the integer-dot GEMV.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg; never by the product path.  It shares no code,
table or constant with the HIP library.

Source: the "Ultra LLM Engine" page says the quantized linear layers quantize
their activations dynamically before the fused GEMV/GEMM (Core Components >
Quantized Model) and names no scheme for them.  The readings taken here:

  R-AQ  symmetric int8 codes per (activation row m, weight group g): with
        a = max |x| over the group's G values (fp32, exact from fp16),
        r = 127 / a rounded to fp32, each code is q = rint(x * r) with the
        product rounded to fp32 and the rint ties-to-even, clamped to
        [-127, 127]; a == 0 gives r = 0 and q = 0.  The activation scale is
        s_x = a / 127 rounded to fp32.  (Both divisions and the product are
        IEEE fp32 operations, so a kernel that performs them in fp32 takes
        the same integer decisions.)
  R-AD  product with the INT weights (w' = q_w * s + z, the INT readings):
        y[m, n] = sum_g s_x[m, g] * (s[n, g] * D + z[n, g] * Q) with
        D = sum over the group of q_w * q_x and Q = sum of q_x, both integer
        and exact, the rest evaluated in fp64.  This is exactly
        sum_k (s_x q_x)[m, k] * w'[n, k]: the dot product of the dequantized
        activations with the dequantized weights.
  NF4 weights carry codebook values, not integers, so the integer-dot path is
  defined for the INT family only.
"""
from __future__ import annotations

import numpy as np

__all__ = ["quantize_activations", "dequant_activations", "gemv_a8_ref", "A8_QMAX"]

A8_QMAX = 127


def quantize_activations(x16: np.ndarray, group: int):
    """(q int8 [m, k], s_x fp32 [m, k/group]) from fp16 x [m, k] (R-AQ)."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float32)
    m, k = x.shape
    if k % group:
        raise ValueError("k must be a multiple of the group size")
    xg = x.reshape(m, k // group, group)
    a = np.abs(xg).max(axis=-1)                                      # fp32, exact
    r = np.zeros_like(a)
    nz = a > 0
    r[nz] = np.float32(A8_QMAX) / a[nz]                              # fp32 division
    prod = (xg * r[..., None]).astype(np.float32)                    # fp32 product
    q = np.clip(np.rint(prod), -A8_QMAX, A8_QMAX).astype(np.int8)   # ties to even
    s_x = (a / np.float32(A8_QMAX)).astype(np.float32)
    return q.reshape(m, k), s_x


def dequant_activations(q: np.ndarray, s_x: np.ndarray, group: int) -> np.ndarray:
    """fp64 s_x * q, the activations the integer path multiplies."""
    m, k = q.shape
    qg = q.astype(np.float64).reshape(m, k // group, group)
    return (qg * s_x.astype(np.float64)[..., None]).reshape(m, k)


def gemv_a8_ref(q_x: np.ndarray, s_x: np.ndarray, q_w: np.ndarray, s16: np.ndarray,
                z16: np.ndarray, group: int) -> np.ndarray:
    """y [m, n] fp64 from activation codes and scales and the INT weight codes
    and (s, z) per group (R-AD): group-wise integer sums, then the scales."""
    m, k = q_x.shape
    n = q_w.shape[0]
    ng = k // group
    xg = q_x.astype(np.int64).reshape(m, ng, group)
    wg = q_w.astype(np.int64).reshape(n, ng, group)
    d = np.einsum("mgk,ngk->mng", xg, wg)                            # exact integers
    qs = xg.sum(axis=-1)                                             # [m, ng]
    s = np.asarray(s16, dtype=np.float16).astype(np.float64)        # [n, ng]
    z = np.asarray(z16, dtype=np.float16).astype(np.float64)
    sx = s_x.astype(np.float64)                                      # [m, ng]
    inner = s[None] * d.astype(np.float64) + z[None] * qs[:, None, :].astype(np.float64)
    return (sx[:, None, :] * inner).sum(axis=-1)
