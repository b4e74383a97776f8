"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds shapes and random draws only -- none of the quantization or
product arithmetic.  Both the oracle and the HIP path receive the arrays it
returns; neither is imported here.

Shapes follow the models the "Ultra LLM Engine" page runs: a small random
decoder (Quick Start: hidden 256) and 4096-wide checkpoints (CLI Examples:
hidden 4096), with 7B-style projection widths (MLP up-projection 11008, wide
MLP 14336, attention 4096).  Weights are N(0, 0.02) drawn in fp64 and rounded
to fp32, optionally with 0.1 % of entries scaled by 20 (outliers); activations
are N(0, 1) rounded to fp16.  The page's own models are randomly initialised
(Quick Start and Current Scope), so random weights stand in faithfully.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    scheme: str          # "int2" | "int4" | "int8" | "nf4"
    group: int
    k: int
    n: int
    ms: tuple            # activation row counts exercised
    outliers: bool = False
    seed: int = 0
    path: str = "gemv"   # "gemv" (M <= 8) or "gemm" (bf16 matrix cores)
    gguf: int = 0        # GGUF block type the weights arrive in (2 Q4_0, 8 Q8_0); 0: fp32 weights
    note: str = field(default="", compare=False)

    @property
    def mmax(self) -> int:
        return max(self.ms)


# The workloads (names say what they are).
WORKLOADS = {
    "int4_g32_k256_n768": Workload(
        "int4_g32_k256_n768", "int4", 32, 256, 768, (1,),
        note="small decoder layer, hidden 256"),
    "int4_g64_k4096_n11008": Workload(
        "int4_g64_k4096_n11008", "int4", 64, 4096, 11008, (1, 4), outliers=True,
        note="7B-style MLP up-projection, decode"),
    "int8_g128_k4096_n4096": Workload(
        "int8_g128_k4096_n4096", "int8", 128, 4096, 4096, (1, 8),
        note="attention q/o projection"),
    "int2_g16_k4096_n4096": Workload(
        "int2_g16_k4096_n4096", "int2", 16, 4096, 4096, (1, 8),
        note="attention q/o projection"),
    "nf4_g64_k4096_n14336": Workload(
        "nf4_g64_k4096_n14336", "nf4", 64, 4096, 14336, (1,),
        note="wide MLP projection"),
    "int4_g128_k4096_n11008_gemm": Workload(
        "int4_g128_k4096_n11008_gemm", "int4", 128, 4096, 11008, (16, 64, 256),
        path="gemm", note="batched decode / prefill"),
    # The same GEMM for the other schemes, on the GEMV workloads' matrices.
    "int8_g128_k4096_n4096_gemm": Workload(
        "int8_g128_k4096_n4096_gemm", "int8", 128, 4096, 4096, (64, 256), seed=1,
        path="gemm", note="attention q/o projection, batched"),
    "int2_g16_k4096_n4096_gemm": Workload(
        "int2_g16_k4096_n4096_gemm", "int2", 16, 4096, 4096, (64, 256), seed=2,
        path="gemm", note="attention q/o projection, batched"),
    "nf4_g64_k4096_n14336_gemm": Workload(
        "nf4_g64_k4096_n14336_gemm", "nf4", 64, 4096, 14336, (64, 256), seed=3,
        path="gemm", note="wide MLP projection, batched"),
    # GGUF blocks (random quant bytes and scales) re-laid into INT4 / INT8 with G = 32.
    "q4_0_k4096_n11008": Workload(
        "q4_0_k4096_n11008", "int4", 32, 4096, 11008, (1, 4), seed=4, gguf=2,
        note="7B-style MLP up-projection from GGUF Q4_0, decode"),
    "q8_0_k4096_n4096": Workload(
        "q8_0_k4096_n4096", "int8", 32, 4096, 4096, (1, 8), seed=5, gguf=8,
        note="attention q/o projection from GGUF Q8_0, decode"),
    "q4_0_k4096_n11008_gemm": Workload(
        "q4_0_k4096_n11008_gemm", "int4", 32, 4096, 11008, (256,), seed=6, gguf=2,
        path="gemm", note="GGUF Q4_0 MLP up-projection, batched"),
}

@dataclass(frozen=True)
class NormRopeWorkload:
    """Fused RMSNorm + RoPE over [tokens, heads, head_dim] fp16 vectors."""
    name: str
    tokens: int
    heads: int
    head_dim: int
    max_pos: int
    sequence: bool = True     # positions 0 .. tokens-1 (prefill) or random (a decode batch)
    theta: float = 10000.0
    eps: float = 1e-6
    seed: int = 0
    note: str = field(default="", compare=False)


NORM_ROPE = {
    "rmsnorm_rope_t4096_h32_d128": NormRopeWorkload(
        "rmsnorm_rope_t4096_h32_d128", 4096, 32, 128, 4096,
        note="prefill of a 4096-wide model, 32 heads of 128"),
    "rmsnorm_rope_t64_h32_d128": NormRopeWorkload(
        "rmsnorm_rope_t64_h32_d128", 64, 32, 128, 4096, sequence=False, seed=1,
        note="one batched decode step, 64 sequences"),
    "rmsnorm_rope_t256_h1_d256": NormRopeWorkload(
        "rmsnorm_rope_t256_h1_d256", 256, 1, 256, 256, seed=2,
        note="small decoder, hidden 256 as one vector"),
}


def make_norm_rope(wl: NormRopeWorkload):
    """x fp16 [T, H, D] ~ N(0, 1); gamma fp32 ~ 1 + 0.1 N(0, 1); positions int32 [T]."""
    rng = np.random.default_rng(wl.seed)
    x = rng.standard_normal((wl.tokens, wl.heads, wl.head_dim)).astype(np.float16)
    gamma = (1.0 + 0.1 * rng.standard_normal(wl.head_dim)).astype(np.float32)
    if wl.sequence:
        pos = np.arange(wl.tokens, dtype=np.int32) % wl.max_pos
    else:
        pos = rng.integers(0, wl.max_pos, wl.tokens).astype(np.int32)
    return x, gamma, pos


# The workload the headline throughput figure is quoted on.
HEADLINE = "int4_g64_k4096_n11008"


def make_weights(n: int, k: int, seed: int = 0, outliers: bool = False,
                 rng: np.random.Generator | None = None) -> np.ndarray:
    """fp32 [n, k] ~ N(0, 0.02); with outliers, 0.1 % of entries (no repeats) x20."""
    rng = np.random.default_rng(seed) if rng is None else rng
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    if outliers:
        idx = rng.choice(n * k, (n * k) // 1000, replace=False)
        w.flat[idx] *= np.float32(20.0)
    return w


def make_x(m: int, k: int, rng: np.random.Generator) -> np.ndarray:
    """fp16 [m, k] ~ N(0, 1)."""
    return rng.standard_normal((m, k)).astype(np.float16)


def make_workload(wl: Workload):
    """(W fp32 [n, k], x fp16 [mmax, k]) from one generator seeded with wl.seed.

    W is drawn first, then the outlier positions, then x; smaller M use the
    first rows of x.
    """
    rng = np.random.default_rng(wl.seed)
    w = make_weights(wl.n, wl.k, outliers=wl.outliers, rng=rng)
    x = make_x(wl.mmax, wl.k, rng)
    return w, x


# Bytes per 32-weight block of the GGUF block formats (a size, not arithmetic).
GGUF_BLOCK_BYTES = {2: 18, 8: 34}


def make_gguf_blocks(gtype: int, n: int, k: int, seed: int = 0, dmax: float = 0.01,
                     rng: np.random.Generator | None = None) -> np.ndarray:
    """GGUF Q4_0 (2) or Q8_0 (8) blocks of an [n, k] matrix, uint8 [n * k/32 * size]:
    uniform random quant bytes after an fp16 scale d ~ N(0, dmax) (either sign)
    stored little-endian in the first two bytes of each block."""
    rng = np.random.default_rng(seed) if rng is None else rng
    size = GGUF_BLOCK_BYTES[gtype]
    blob = rng.integers(0, 256, size=(n, k // 32, size)).astype(np.uint8)
    d = (rng.standard_normal((n, k // 32)) * dmax).astype(np.float16).view(np.uint16)
    blob[..., 0], blob[..., 1] = d & 0xFF, d >> 8
    return blob.reshape(-1)


def make_gguf_workload(wl: Workload):
    """(GGUF blocks of W [n, k], x fp16 [mmax, k]) from one generator seeded with wl.seed."""
    rng = np.random.default_rng(wl.seed)
    blob = make_gguf_blocks(wl.gguf, wl.n, wl.k, rng=rng)
    x = make_x(wl.mmax, wl.k, rng)
    return blob, x


def make_random(n: int, k: int, m: int, seed: int, outliers: bool = False):
    """Small seeded case for parity sweeps: (W fp32 [n, k], x fp16 [m, k])."""
    rng = np.random.default_rng(seed)
    w = make_weights(n, k, outliers=outliers, rng=rng)
    x = make_x(m, k, rng)
    return w, x
