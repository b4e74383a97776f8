"""Each pin must fail when a plausible mistake is planted in the oracle (CPU only).

The mistakes are planted in a copy of the oracle's function table; the oracle
module itself is untouched.
"""
import types

import numpy as np
import pytest

import oracle as o
from tests import pins


def mutant(**overrides):
    ns = types.SimpleNamespace(**{name: getattr(o, name) for name in o.__all__})
    for k, v in overrides.items():
        setattr(ns, k, v)
    return ns


def dequant_drop_zero(q, s16, z16, group):
    return o.dequant_int(q, s16, np.zeros_like(z16), group)


def dequant_zero_sign(q, s16, z16, group):
    return o.dequant_int(q, s16, -z16, group)


def quantize_wrong_qmax(w, bits, group):
    # divides the span by 2^b instead of 2^b - 1
    n, k = w.shape
    wg = w.reshape(n, k // group, group)
    mn, mx = wg.min(2), wg.max(2)
    s16 = ((mx - mn) / np.float32(1 << bits)).astype(np.float16)
    z16 = mn.astype(np.float16)
    q = np.clip(np.rint((wg - z16[..., None].astype(np.float64)) / s16[..., None]), 0,
                (1 << bits) - 1)
    return q.astype(np.uint8).reshape(n, k), s16, z16


def quantize_truncating(w, bits, group):
    # floor instead of round-to-nearest for the code
    q, s16, z16 = o.quantize_int(w, bits, group)
    n, k = w.shape
    wg = w.reshape(n, k // group, group).astype(np.float64)
    d = (wg - z16.astype(np.float64)[..., None]) / s16.astype(np.float64)[..., None]
    q2 = np.clip(np.floor(d), 0, (1 << bits) - 1)
    return q2.astype(np.uint8).reshape(n, k), s16, z16


def pack_high_first(q, bits):
    n, k = q.shape
    per = 8 // bits
    qq = q.astype(np.uint32).reshape(n, k // per, per)[:, :, ::-1]
    return o.pack_codes(qq.reshape(n, k).astype(np.uint8), bits)


def quantize_nf4_ties_up(w, group=64, codebook=None):
    c = o.nf4_codebook()
    n, k = w.shape
    wg = w.reshape(n, k // group, group)
    a16 = np.abs(wg).max(2).astype(np.float16)
    v = wg.astype(np.float64) / a16.astype(np.float64)[..., None]
    mid = (c[:-1].astype(np.float64) + c[1:].astype(np.float64)) / 2
    q = np.searchsorted(mid, v.reshape(-1), side="right").reshape(v.shape)
    return q.astype(np.uint8).reshape(n, k), a16


def codebook_symmetric():
    # a plausible wrong table: symmetric quantiles, no exact zero
    c = o.nf4_codebook().copy()
    c[:8] = -c[8:][::-1]
    return c


def gemv_transposed_rows(x16, wdq):
    return (x16.astype(np.float64) @ wdq.astype(np.float64).T)[:, ::-1]


def gemv_fp32(x16, wdq):
    return (x16.astype(np.float32) @ wdq.astype(np.float32).T).astype(np.float64)


def gemm_no_x_cast(x16, wdq):
    return x16.astype(np.float64) @ o.bf16_rne(wdq).astype(np.float64).T


def bf16_truncate(a):
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return (u & np.uint32(0xFFFF0000)).view(np.float32)


def rope_interleaved(x16, gamma, pos, cos, sin, eps):
    # pairs (2i, 2i+1) instead of (i, i + D/2)
    y = o.rmsnorm_rope(x16, gamma, np.zeros_like(pos), cos, sin, eps)
    c = cos[pos].astype(np.float64)[:, None, :]
    s = sin[pos].astype(np.float64)[:, None, :]
    a, b = y[..., 0::2], y[..., 1::2]
    out = np.empty_like(y)
    out[..., 0::2], out[..., 1::2] = a * c - b * s, b * c + a * s
    return out


def rope_sin_flipped(x16, gamma, pos, cos, sin, eps):
    return o.rmsnorm_rope(x16, gamma, pos, cos, -sin, eps)


def rmsnorm_sum(x16, gamma, pos, cos, sin, eps):
    # sum of squares instead of the mean
    d = x16.shape[-1]
    return o.rmsnorm_rope(x16, gamma, pos, cos, sin, eps) / np.sqrt(d)


def rmsnorm_eps_outside(x16, gamma, pos, cos, sin, eps):
    x = x16.astype(np.float64)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True))
    xr = x / (r + np.float64(np.float32(eps))) * r / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + 0.0)
    return o.rmsnorm_rope(xr, gamma, pos, cos, sin, 0.0) * (r / (r + np.float64(np.float32(eps))))


def rope_gamma_after(x16, gamma, pos, cos, sin, eps):
    y = o.rmsnorm_rope(x16, np.ones_like(gamma), pos, cos, sin, eps)
    return y * np.asarray(gamma, np.float64)


def rope_table_wrong_exponent(theta, d, max_pos):
    i = np.arange(d // 2, dtype=np.float64)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * (theta ** (-i / d))[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def a8_per_row_scale(x16, group):
    # one scale for the whole activation row instead of one per group
    x = np.asarray(x16, dtype=np.float16).astype(np.float32)
    m, k = x.shape
    a = np.abs(x).max(axis=1, keepdims=True)
    r = np.where(a > 0, np.float32(127) / np.where(a > 0, a, 1), 0).astype(np.float32)
    q = np.clip(np.rint((x * r).astype(np.float32)), -127, 127).astype(np.int8)
    s = np.repeat((a / np.float32(127)).astype(np.float32), k // group, axis=1)
    return q, s


def a8_qmax_128(x16, group):
    x = np.asarray(x16, dtype=np.float16).astype(np.float32)
    m, k = x.shape
    xg = x.reshape(m, k // group, group)
    a = np.abs(xg).max(axis=-1)
    r = np.where(a > 0, np.float32(128) / np.where(a > 0, a, 1), 0).astype(np.float32)
    q = np.clip(np.rint((xg * r[..., None]).astype(np.float32)), -127, 127).astype(np.int8)
    return q.reshape(m, k), (a / np.float32(128)).astype(np.float32)


def a8_floor(x16, group):
    x = np.asarray(x16, dtype=np.float16).astype(np.float32)
    m, k = x.shape
    xg = x.reshape(m, k // group, group)
    a = np.abs(xg).max(axis=-1)
    r = np.where(a > 0, np.float32(127) / np.where(a > 0, a, 1), 0).astype(np.float32)
    q = np.clip(np.floor((xg * r[..., None]).astype(np.float32)), -127, 127).astype(np.int8)
    return q.reshape(m, k), (a / np.float32(127)).astype(np.float32)


def a8_drop_zero_term(q_x, s_x, q_w, s16, z16, group):
    return o.gemv_a8_ref(q_x, s_x, q_w, s16, np.zeros_like(z16), group)


def a8_scale_by_next_group(q_x, s_x, q_w, s16, z16, group):
    # activation scales taken one group off
    return o.gemv_a8_ref(q_x, np.roll(s_x, 1, axis=1), q_w, s16, z16, group)



def gguf_q4_consecutive_nibbles(blob, gtype, n, k):
    # value 2j in the low nibble of byte j, 2j+1 in the high (the INT4 order)
    if gtype != 2:
        return o.decode_gguf(blob, gtype, n, k)
    b = np.asarray(blob, np.uint8).reshape(n, k // 32, 18)
    d = (b[..., 0].astype(np.uint16) | (b[..., 1].astype(np.uint16) << 8)).view(np.float16)
    qs = b[..., 2:].astype(np.int64)
    v = np.stack([qs & 15, qs >> 4], axis=-1).reshape(n, k // 32, 32) - 8
    return (v * d.astype(np.float64)[..., None]).reshape(n, k)


def gguf_q4_no_offset(blob, gtype, n, k):
    w = o.decode_gguf(blob, gtype, n, k)
    if gtype != 2:
        return w
    b = np.asarray(blob, np.uint8).reshape(n, k // 32, 18)
    d = (b[..., 0].astype(np.uint16) | (b[..., 1].astype(np.uint16) << 8)).view(np.float16)
    return w + np.repeat(8.0 * d.astype(np.float64), 32, axis=1)


def gguf_q8_unsigned(blob, gtype, n, k):
    if gtype != 8:
        return o.decode_gguf(blob, gtype, n, k)
    b = np.asarray(blob, np.uint8).reshape(n, k // 32, 34)
    d = (b[..., 0].astype(np.uint16) | (b[..., 1].astype(np.uint16) << 8)).view(np.float16)
    return (b[..., 2:].astype(np.float64) * d.astype(np.float64)[..., None]).reshape(n, k)


def gguf_scale_big_endian(blob, gtype, n, k):
    size = 18 if gtype == 2 else 34
    b = np.asarray(blob, np.uint8).reshape(-1, size).copy()
    b[:, [0, 1]] = b[:, [1, 0]]
    return o.decode_gguf(b.reshape(-1), gtype, n, k)


def gguf_as_int_zero_off_by_one(blob, gtype, n, k):
    q, s16, z16 = o.gguf_as_int(blob, gtype, n, k)
    return q, s16, (z16.astype(np.float64) + s16.astype(np.float64)).astype(np.float16)


def gguf_as_int_no_bias(blob, gtype, n, k):
    # Q8_0 bytes taken as unsigned codes with the -128 d zero point kept
    q, s16, z16 = o.gguf_as_int(blob, gtype, n, k)
    if gtype == 8:
        q = (q.astype(np.int64) - 128).astype(np.uint8)
    return q, s16, z16

CASES = [
    ("dequant drops the zero term", dict(dequant_int=dequant_drop_zero),
     lambda ns: pins.check_grid_recovery(ns, 4, 64)),
    ("dequant flips the zero sign", dict(dequant_int=dequant_zero_sign),
     lambda ns: pins.check_packing_golden(ns)),
    ("scale divides by 2^b", dict(quantize_int=quantize_wrong_qmax),
     lambda ns: pins.check_grid_recovery(ns, 4, 32)),
    ("code truncates", dict(quantize_int=quantize_truncating),
     lambda ns: pins.check_roundtrip_int(
         ns, (np.random.default_rng(0).standard_normal((8, 256)) * .02).astype(np.float32), 4, 64)),
    ("high nibble first", dict(pack_codes=pack_high_first),
     lambda ns: pins.check_packing_golden(ns)),
    ("NF4 ties go up", dict(quantize_nf4=quantize_nf4_ties_up),
     lambda ns: pins.check_nearest_bruteforce(ns)),
    ("symmetric codebook", dict(nf4_codebook=codebook_symmetric),
     lambda ns: pins.check_codebook(ns)),
    ("GEMV output columns reversed", dict(gemv_ref=gemv_transposed_rows),
     lambda ns: pins.check_products_exact(ns)),
    ("GEMV in fp32", dict(gemv_ref=gemv_fp32),
     lambda ns: pins.check_products_exact(ns, k=64)),
    ("GEMM skips the bf16 cast of x", dict(gemm_ref=gemm_no_x_cast),
     lambda ns: pins.check_products_exact(ns)),
    ("bf16 truncates", dict(bf16_rne=bf16_truncate),
     lambda ns: pins.check_bf16(ns)),
    ("RoPE pairs neighbours", dict(rmsnorm_rope=rope_interleaved),
     lambda ns: pins.check_rope_bruteforce(ns)),
    ("RoPE turns the wrong way", dict(rmsnorm_rope=rope_sin_flipped),
     lambda ns: pins.check_rope_bruteforce(ns)),
    ("RMSNorm uses the sum", dict(rmsnorm_rope=rmsnorm_sum),
     lambda ns: pins.check_rmsnorm_identity(ns)),
    ("RMSNorm adds eps outside the root", dict(rmsnorm_rope=rmsnorm_eps_outside),
     lambda ns: pins.check_rmsnorm_identity(ns)),
    ("RMSNorm gain applied after RoPE", dict(rmsnorm_rope=rope_gamma_after),
     lambda ns: pins.check_rope_bruteforce(ns)),
    ("RoPE frequencies theta^(-i/D)", dict(rope_table=rope_table_wrong_exponent),
     lambda ns: pins.check_rope_table(ns)),
    ("A8 one scale per row", dict(quantize_activations=a8_per_row_scale),
     lambda ns: pins.check_a8_grid(ns)),
    ("A8 scale 128", dict(quantize_activations=a8_qmax_128),
     lambda ns: pins.check_a8_grid(ns)),
    ("A8 floor codes", dict(quantize_activations=a8_floor),
     lambda ns: pins.check_a8_roundtrip(ns)),
    ("A8 drops the zero term", dict(gemv_a8_ref=a8_drop_zero_term),
     lambda ns: pins.check_a8_products(ns)),
    ("A8 scales one group off", dict(gemv_a8_ref=a8_scale_by_next_group),
     lambda ns: pins.check_a8_bruteforce(ns)),
    ("GGUF Q4_0 nibbles in INT4 order", dict(decode_gguf=gguf_q4_consecutive_nibbles),
     lambda ns: pins.check_gguf_placement(ns)),
    ("GGUF Q4_0 without the -8", dict(decode_gguf=gguf_q4_no_offset),
     lambda ns: pins.check_gguf_golden(ns)),
    ("GGUF Q8_0 bytes unsigned", dict(decode_gguf=gguf_q8_unsigned),
     lambda ns: pins.check_gguf_golden(ns)),
    ("GGUF scale big-endian", dict(decode_gguf=gguf_scale_big_endian),
     lambda ns: pins.check_gguf_golden(ns)),
    ("GGUF INT form zero point one step off", dict(gguf_as_int=gguf_as_int_zero_off_by_one),
     lambda ns: pins.check_gguf_int_form(ns)),
    ("GGUF INT form Q8_0 codes not biased", dict(gguf_as_int=gguf_as_int_no_bias),
     lambda ns: pins.check_gguf_int_form(ns)),
]


@pytest.mark.parametrize("label,over,check", CASES, ids=[c[0] for c in CASES])
def test_planted_mistake_is_caught(label, over, check):
    with pytest.raises(AssertionError):
        check(mutant(**over))
