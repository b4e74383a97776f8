"""Plain, slow, obviously-correct CPU oracle for the quantized linear-layer hot path.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the CPU-baseline
leg of the benchmark; never by the product path.  It shares no code, table or
constant with the HIP library.

What it computes (source: the "Ultra LLM Engine" page):
  * Core Components > Quantization, scheme table: an ``int`` family
    (group-wise asymmetric uniform quantization with 2, 4 or 8 bits) and an
    ``nf4`` family (NormalFloat4 with the QLoRA codebook); both pack several
    low-bit codes into each byte and come with matching dequantizers.
  * Core Components > Fused Kernels: the fused layer multiplies activations by
    the dequantized weight, as a GEMV for single-token decode and as a GEMM
    for batched decode.
  * Core Components > Quantized Model: linear layers hold their weights in
    this quantized form (QuantLinear).

The page fixes the families, not the arithmetic.  Every step below that the
page leaves open is a *reading*; each is named where it is used:

  R-Z1  zero point = the real value that code 0 maps to (z = group minimum),
        so w' = q*s + z; scale s = (max - min) / (2^b - 1).
  R-S2  s is formed with two fp32 operations (subtract, divide), then rounded
        to fp16 (round to nearest even); z = fp16(min).
  R-S3  the code is rint((w - z) / s) evaluated in fp64, ties to even,
        clamped to [0, 2^b - 1]; a group whose fp16 scale is 0 gets q = 0.
  R-DQ  dequantized weight w' = fp32_round(q*s + z); the product and sum are
        exact in fp64, so the value is rounded exactly once.
  R-NF  NF4: a = fp16(max |w|) per group of 64; v = w / a in fp64; q = index
        of the nearest codebook entry, a value exactly on a midpoint taking the
        lower index; a == 0 gives q = 7 (the entry 0.0); w' = fp32(C[q] * a).
  R-CB  codebook: QLoRA's NormalFloat construction with p* = 0.9677083
        (8 positive quantiles, 7 negative, and 0; normalised to [-1, 1]).
  R-PK  packing: INT4/NF4 two codes per byte, low nibble first; INT2 four
        codes per byte, lowest bits first; INT8 one code per byte.  INT params
        are (s, z) fp16 pairs per group, interleaved [n, k/G, 2]; NF4 params are
        one fp16 absmax per group [n, k/64].
  R-Y   GEMV:  y = x . w'^T in fp64 from fp16 x.
        GEMM (bf16 matrix-core path): y = bf16(x) . bf16(w')^T in fp64, both
        casts round-to-nearest-even from fp32.
"""
from __future__ import annotations

from fractions import Fraction
from statistics import NormalDist

import numpy as np

__all__ = [
    "SCHEMES", "BITS", "QMAX", "GROUPS", "nf4_codebook", "quantize_int",
    "dequant_int", "quantize_nf4", "dequant_nf4", "pack_codes", "unpack_codes",
    "pack_params_int", "unpack_params_int", "pack_params_nf4",
    "unpack_params_nf4", "quantize_pack", "dequant_packed", "gemv_ref",
    "bf16_rne", "gemm_ref", "NF4_PSTAR",
]

# Scheme names and widths (Ultra LLM Engine, Highlights table, Quantization
# row: INT-2, INT-4, INT-8 and NF4).
SCHEMES = ("int2", "int4", "int8", "nf4")
BITS = {"int2": 2, "int4": 4, "int8": 8, "nf4": 4}
QMAX = {2: 3, 4: 15, 8: 255}
# Group sizes the path supports (reading: the page names no group size).
GROUPS = {"int2": (16, 32, 64, 128), "int4": (32, 64, 128),
          "int8": (32, 64, 128), "nf4": (64,)}

NF4_PSTAR = 0.9677083


# ---------------------------------------------------------------------------
# NF4 codebook (reading R-CB)
# ---------------------------------------------------------------------------
def nf4_codebook(pstar: float = NF4_PSTAR) -> np.ndarray:
    """The 16-level NormalFloat codebook as fp32, built from the inverse normal CDF.

    Ultra LLM Engine, Core Components > Quantization, ``nf4`` row: a QLoRA-style
    codebook.  The page prints no values.  Construction (QLoRA, Dettmers et
    al. 2023, NormalFloat section): take the standard-normal quantiles at 8
    equally spaced probabilities from p* down to 0.5 (0.5 itself excluded) for
    the positive half and at 7 such probabilities for the negative half, add an
    exact 0, sort, and divide by the largest quantile so the range is [-1, 1].
    """
    inv = NormalDist().inv_cdf
    pos = [inv(p) for p in np.linspace(pstar, 0.5, 9)[:-1]]
    neg = [-inv(p) for p in np.linspace(pstar, 0.5, 8)[:-1]]
    vals = np.array(sorted(pos + [0.0] + neg), dtype=np.float64)
    return (vals / inv(pstar)).astype(np.float32)


# ---------------------------------------------------------------------------
# Group-wise asymmetric INT-N (readings R-Z1, R-S2, R-S3, R-DQ)
# ---------------------------------------------------------------------------
def _groups(w: np.ndarray, group: int) -> np.ndarray:
    n, k = w.shape
    if k % group:
        raise ValueError(f"k={k} is not a multiple of the group size {group}")
    return w.reshape(n, k // group, group)


def quantize_int(w: np.ndarray, bits: int, group: int):
    """Group-wise asymmetric uniform quantization of an fp32 [n, k] matrix.

    Ultra LLM Engine, Core Components > Quantization, ``int`` row (asymmetric,
    uniform, group-wise, 2/4/8 bits).  Per row n and group g (G consecutive
    columns): scale s = (max - min)/qmax, zero z = min, code
    q = clamp(round((w - z)/s), 0, qmax).

    Returns (q uint8 [n, k], s16 float16 [n, k/G], z16 float16 [n, k/G]).
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    qmax = QMAX[bits]
    wg = _groups(w, group)
    mn = wg.min(axis=2)                      # exact (fp32 values)
    mx = wg.max(axis=2)
    span32 = (mx - mn).astype(np.float32)    # one fp32 subtraction, RNE
    s32 = (span32 / np.float32(qmax)).astype(np.float32)  # one fp32 division
    s16 = s32.astype(np.float16)             # fp32 -> fp16, RNE
    z16 = mn.astype(np.float16)
    s64 = s16.astype(np.float64)[..., None]
    z64 = z16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        d = (wg.astype(np.float64) - z64) / s64
    q = np.clip(np.rint(d), 0, qmax)         # rint: round half to even
    q = np.where(s64 == 0.0, 0.0, q)         # constant group: all codes 0
    return q.astype(np.uint8).reshape(w.shape), s16, z16


def dequant_int(q: np.ndarray, s16: np.ndarray, z16: np.ndarray, group: int):
    """w' = fp32(q*s + z), evaluated exactly in fp64 and rounded once (R-DQ)."""
    n, k = q.shape
    qg = q.reshape(n, k // group, group).astype(np.float64)
    w = qg * s16.astype(np.float64)[..., None] + z16.astype(np.float64)[..., None]
    return w.astype(np.float32).reshape(n, k)


# ---------------------------------------------------------------------------
# NF4 (reading R-NF)
# ---------------------------------------------------------------------------
def quantize_nf4(w: np.ndarray, group: int = 64, codebook: np.ndarray | None = None):
    """NormalFloat4 quantization with a per-group fp16 absmax.

    Ultra LLM Engine, Core Components > Quantization, ``nf4`` row.  Per group:
    a = fp16(max|w|); v = w/a; q = nearest codebook entry (midpoint -> lower
    index).  Returns (q uint8 [n, k], a16 float16 [n, k/G]).
    """
    c = nf4_codebook() if codebook is None else codebook
    w = np.ascontiguousarray(w, dtype=np.float32)
    wg = _groups(w, group)
    a16 = np.abs(wg).max(axis=2).astype(np.float16)
    a64 = a16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        v = wg.astype(np.float64) / a64
    # Midpoints between neighbouring entries, exact in fp64.  The nearest entry
    # is the number of midpoints strictly below v; a tie stays at the lower one.
    mid = (c[:-1].astype(np.float64) + c[1:].astype(np.float64)) / 2.0
    q = np.searchsorted(mid, v.reshape(-1), side="left").reshape(v.shape)
    q = np.where(a64 == 0.0, 7, q)
    return q.astype(np.uint8).reshape(w.shape), a16


def dequant_nf4(q: np.ndarray, a16: np.ndarray, group: int = 64,
                codebook: np.ndarray | None = None):
    """w' = fp32(C[q] * a); the fp64 product is exact, so one rounding."""
    c = nf4_codebook() if codebook is None else codebook
    n, k = q.shape
    cq = c.astype(np.float64)[q.reshape(n, k // group, group)]
    return (cq * a16.astype(np.float64)[..., None]).astype(np.float32).reshape(n, k)


# ---------------------------------------------------------------------------
# Bit packing (reading R-PK; the page says only that several low-bit values
# share a byte: Core Components > Quantization)
# ---------------------------------------------------------------------------
def pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """Codes [n, k] -> bytes [n, k*bits/8]; the first code of a byte sits in its lowest bits."""
    n, k = q.shape
    per = 8 // bits
    if k % per:
        raise ValueError("k does not fill whole bytes")
    q = q.astype(np.uint32).reshape(n, k // per, per)
    out = np.zeros((n, k // per), dtype=np.uint32)
    for i in range(per):
        out |= q[:, :, i] << (bits * i)
    return out.astype(np.uint8)


def unpack_codes(codes: np.ndarray, bits: int, k: int) -> np.ndarray:
    """Inverse of :func:`pack_codes`."""
    n = codes.shape[0]
    per = 8 // bits
    c = codes.astype(np.uint32).reshape(n, k // per)
    mask = (1 << bits) - 1
    out = np.stack([(c >> (bits * i)) & mask for i in range(per)], axis=2)
    return out.reshape(n, k).astype(np.uint8)


def pack_params_int(s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """(s, z) fp16 bit patterns interleaved per group: uint16 [n, k/G, 2]."""
    return np.stack([s16.view(np.uint16), z16.view(np.uint16)], axis=-1)


def unpack_params_int(params: np.ndarray):
    p = params.view(np.uint16)
    return p[..., 0].view(np.float16), p[..., 1].view(np.float16)


def pack_params_nf4(a16: np.ndarray) -> np.ndarray:
    return a16.view(np.uint16).copy()


def unpack_params_nf4(params: np.ndarray):
    return params.view(np.uint16).view(np.float16)


def quantize_pack(w: np.ndarray, scheme: str, group: int):
    """Quantize an fp32 [n, k] matrix and pack it: (codes uint8, params uint16)."""
    bits = BITS[scheme]
    if scheme == "nf4":
        q, a16 = quantize_nf4(w, group)
        return pack_codes(q, bits), pack_params_nf4(a16)
    q, s16, z16 = quantize_int(w, bits, group)
    return pack_codes(q, bits), pack_params_int(s16, z16)


def dequant_packed(codes: np.ndarray, params: np.ndarray, scheme: str,
                   group: int, k: int) -> np.ndarray:
    """Unpack and dequantize packed weights to fp32 [n, k]."""
    bits = BITS[scheme]
    q = unpack_codes(codes, bits, k)
    if scheme == "nf4":
        return dequant_nf4(q, unpack_params_nf4(params), group)
    s16, z16 = unpack_params_int(params)
    return dequant_int(q, s16, z16, group)


# ---------------------------------------------------------------------------
# Products (reading R-Y; Ultra LLM Engine, Core Components > Fused Kernels)
# ---------------------------------------------------------------------------
def gemv_ref(x16: np.ndarray, wdq: np.ndarray) -> np.ndarray:
    """y[m, n] = sum_k x[m, k] * w'[n, k], fp64 (fp16 activation path)."""
    return x16.astype(np.float64) @ wdq.astype(np.float64).T


def bf16_rne(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even); returned as fp32.

    bfloat16 keeps the upper 16 bits of an fp32 word.  Adding 0x7FFF plus the
    lowest kept bit before truncating rounds to nearest with ties to even.
    Inputs here are finite, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (r << 16).astype(np.uint32).view(np.float32)


def gemm_ref(x16: np.ndarray, wdq: np.ndarray) -> np.ndarray:
    """y = bf16(x) . bf16(w')^T in fp64 (bf16 matrix-core path)."""
    xb = bf16_rne(x16.astype(np.float32)).astype(np.float64)
    wb = bf16_rne(wdq).astype(np.float64)
    return xb @ wb.T
