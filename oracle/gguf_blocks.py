"""Plain CPU oracle for GGUF Q4_0 and Q8_0 weight blocks.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg; never by the product path.  It shares no code,
table or constant with the HIP library.

Source: the "Ultra LLM Engine" page puts dequantizers for the common GGUF
block formats Q4_0 and Q8_0 on its roadmap (Roadmap Ideas) and has its GGUF
loader detect such tensors and refuse them loudly (Checkpoint Loading); the
lollm page's shared infrastructure dequantizes GGUF blocks itself (model
table notes, Shared infra).  Neither page prints the block layout.  Reading
R-GG takes it from the public GGUF format definition:

  * a weight row of k values is split into k/32 blocks of 32 consecutive
    values; rows follow one another, blocks follow one another in a row;
  * Q4_0 block, 18 bytes: an IEEE fp16 scale d (little-endian), then 16
    bytes; byte j carries value j in its low four bits and value j + 16 in
    its high four bits; each value is (nibble - 8) * d;
  * Q8_0 block, 34 bytes: an fp16 scale d, then 32 signed bytes q; each
    value is q * d.

Every value above is a product of a small integer and an fp16 number, so it
is exact in fp32; the oracle forms it in fp64.

R-GI (the same weights in the INT form w' = q * s + z with G = 32): Q4_0 is
q = nibble, s = d, z = -8 d; Q8_0 is q = byte + 128 (as unsigned), s = d,
z = -128 d.  z is exact in fp16 unless it overflows; a non-finite d or an
overflowing z is refused, never guessed (the lollm page, Vision, item 3; the
Ultra LLM Engine loader's loud refusal).
The INT form reproduces every value exactly as a number (a zero may change
sign: (nibble - 8) * d is -0 where nibble * d - 8 d is +0).
"""
from __future__ import annotations

import numpy as np

__all__ = ["GGUF_Q4_0", "GGUF_Q8_0", "GGUF_BLOCK", "GGUF_BLOCK_BYTES",
           "decode_gguf", "gguf_as_int"]

# GGUF tensor type ids of the two block formats (the file format's own ids).
GGUF_Q4_0 = 2
GGUF_Q8_0 = 8
GGUF_BLOCK = 32
GGUF_BLOCK_BYTES = {GGUF_Q4_0: 18, GGUF_Q8_0: 34}


def _blocks(blob: np.ndarray, gtype: int, n: int, k: int) -> np.ndarray:
    if gtype not in GGUF_BLOCK_BYTES:
        raise ValueError(f"unknown GGUF block type {gtype}")
    if k % GGUF_BLOCK:
        raise ValueError("k must be a multiple of 32")
    b = np.asarray(blob, dtype=np.uint8).reshape(-1)
    nb = GGUF_BLOCK_BYTES[gtype]
    if b.size != n * (k // GGUF_BLOCK) * nb:
        raise ValueError("blob size does not match n, k")
    return b.reshape(n, k // GGUF_BLOCK, nb)


def _scales(blk: np.ndarray) -> np.ndarray:
    """fp16 d of every block (little-endian bytes 0 and 1) as uint16 bits."""
    return blk[..., 0].astype(np.uint16) | (blk[..., 1].astype(np.uint16) << 8)


def _codes(blk: np.ndarray, gtype: int) -> np.ndarray:
    """The 32 integer values of every block, in weight order (R-GG)."""
    if gtype == GGUF_Q4_0:
        qs = blk[..., 2:18]
        low = (qs & 0x0F).astype(np.int64)          # values 0 .. 15 of the block
        high = (qs >> 4).astype(np.int64)           # values 16 .. 31
        return np.concatenate([low, high], axis=-1) - 8
    return blk[..., 2:34].view(np.int8).astype(np.int64)


def decode_gguf(blob: np.ndarray, gtype: int, n: int, k: int) -> np.ndarray:
    """W [n, k] fp64 from GGUF Q4_0 / Q8_0 blocks (R-GG)."""
    blk = _blocks(blob, gtype, n, k)
    d = _scales(blk).view(np.float16).astype(np.float64)        # [n, k/32]
    v = _codes(blk, gtype).astype(np.float64) * d[..., None]    # [n, k/32, 32]
    return v.reshape(n, k)


def gguf_as_int(blob: np.ndarray, gtype: int, n: int, k: int):
    """(q uint8 [n, k], s fp16 [n, k/32], z fp16 [n, k/32]) of R-GI.

    Raises ValueError for a non-finite d or a zero point beyond fp16."""
    blk = _blocks(blob, gtype, n, k)
    d16 = _scales(blk).view(np.float16)
    d = d16.astype(np.float64)
    if not np.isfinite(d).all():
        raise ValueError("a block scale is NaN or infinite")
    offset = 8 if gtype == GGUF_Q4_0 else 128
    z = -offset * d                                             # exact: power-of-two multiple
    if (np.abs(z) > 65504.0).any():
        raise ValueError("a zero point -offset * d exceeds the fp16 range")
    q = (_codes(blk, gtype) + offset).astype(np.uint8).reshape(n, k)
    return q, d16.copy(), z.astype(np.float16)
