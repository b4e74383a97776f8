"""Checks that pin the oracle to facts outside itself.

Each check takes an object ``o`` exposing the oracle's functions, so the
mutation tests can hand in a copy with one step deliberately broken (on the
CPU) and confirm the check then fails.  Sources for each fact are given per
check; see ``oracle/uq_oracle.py`` for the readings R-* they refer to.
"""
from __future__ import annotations

import os
import re
from fractions import Fraction

import numpy as np

import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# Golden fixture parsing
# ---------------------------------------------------------------------------
def load_packing_cases():
    """Parse tests/golden/packing_handbuilt.txt into a list of case dicts."""
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "packing_handbuilt.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("case "):
                _, name, scheme, g, n, k = line.split()
                cur = dict(name=name, scheme=scheme, group=int(g[2:]),
                           n=int(n[2:]), k=int(k[2:]), w={}, codes={}, params={})
                cases.append(cur)
                continue
            key, val = line.split(":", 1)
            m = re.fullmatch(r"(w|codes|params)(\d+)", key)
            kind, row = m.group(1), int(m.group(2))
            if kind == "w":
                cur["w"][row] = val.strip()
            elif kind == "codes":
                cur["codes"][row] = bytes(int(b, 16) for b in val.split())
            else:
                cur["params"][row] = [int(p, 16) for p in val.split()]
    return cases


def build_case_weights(case, codebook):
    """Evaluate the per-row recipes of a golden case into an fp32 [n, k] matrix."""
    n, k = case["n"], case["k"]
    w = np.zeros((n, k), dtype=np.float64)
    for r in range(n):
        expr = case["w"][r]
        for col in range(k):
            w[r, col] = eval(expr, {"__builtins__": {}},  # own fixture file
                             {"k": col, "C": [float(c) for c in codebook]})
    w32 = w.astype(np.float32)
    assert np.array_equal(w32.astype(np.float64), w), "recipe not exact in fp32"
    return w32


# ---------------------------------------------------------------------------
# P1: bit-exact packing on hand-built matrices
# ---------------------------------------------------------------------------
def check_packing_golden(o):
    """Quantize + pack each hand-built case; bytes and params must equal the fixture.

    Source: Ultra LLM Engine, Core Components > Quantization (codes packed into
    bytes); the expected bytes are derived by hand in the fixture file.
    """
    cb = o.nf4_codebook()
    for case in load_packing_cases():
        w = build_case_weights(case, cb)
        bits = o.BITS[case["scheme"]]
        if case["scheme"] == "nf4":
            q, a16 = o.quantize_nf4(w, case["group"])
            params = o.pack_params_nf4(a16)
            wdq = o.dequant_nf4(q, a16, case["group"])
        else:
            q, s16, z16 = o.quantize_int(w, bits, case["group"])
            params = o.pack_params_int(s16, z16)
            wdq = o.dequant_int(q, s16, z16, case["group"])
        codes = o.pack_codes(q, bits)
        for r in range(case["n"]):
            assert codes[r].tobytes() == case["codes"][r], (case["name"], r, codes[r].tobytes().hex())
            got = [int(v) for v in np.asarray(params[r]).reshape(-1)]
            assert got == case["params"][r], (case["name"], r, [hex(v) for v in got])
        # every weight of these cases lies on the grid: dequant must return it
        assert np.array_equal(wdq, w), case["name"]
        # unpacking returns the codes
        assert np.array_equal(o.unpack_codes(codes, bits, case["k"]), q), case["name"]


# ---------------------------------------------------------------------------
# Exact grid recovery: W = q*s + z built from known q, s, z
# ---------------------------------------------------------------------------
def check_grid_recovery(o, bits, group, seed=0, n=6, k=None):
    """Weights built exactly on a known grid are recovered exactly.

    Source: Ultra LLM Engine, Core Components > Quantization, ``int`` row
    (asymmetric uniform group-wise quantization).  With s = 2^-e, a dyadic z
    and each group holding both code 0 and code qmax, the scale
    (max - min)/qmax is s, the zero (min) is z, every division is exact, and
    so quantize must return (q, s, z) and dequant must return W.
    """
    rng = np.random.default_rng(seed)
    k = k or 4 * group
    qmax = (1 << bits) - 1
    g = k // group
    q = rng.integers(0, qmax + 1, size=(n, g, group))
    perm = rng.permuted(np.tile(np.arange(group), (n, g, 1)), axis=2)
    np.put_along_axis(q, perm[..., :1], 0, axis=2)       # code 0 somewhere
    np.put_along_axis(q, perm[..., 1:2], qmax, axis=2)   # code qmax somewhere
    e = rng.integers(3, 11, size=(n, g))
    s = np.ldexp(1.0, -e)
    z = rng.integers(-1023, 1024, size=(n, g)) * 2.0 ** -10
    w64 = q * s[..., None] + z[..., None]
    w = w64.astype(np.float32).reshape(n, k)
    assert np.array_equal(w.astype(np.float64).reshape(n, g, group), w64)
    q2, s16, z16 = o.quantize_int(w, bits, group)
    assert np.array_equal(q2.reshape(n, g, group), q.astype(np.uint8)), "codes"
    assert np.array_equal(s16.astype(np.float64), s), "scale"
    assert np.array_equal(z16.astype(np.float64), z), "zero"
    assert np.array_equal(o.dequant_int(q2, s16, z16, group), w), "dequant"


# ---------------------------------------------------------------------------
# P2: round-trip error bound
# ---------------------------------------------------------------------------
def check_roundtrip_int(o, w, bits, group):
    """|w' - w| <= s/2 plus half an fp32 ulp of w' (rounding of w').

    Follows from rounding (w - z)/s to the nearest integer code; constant
    groups (s = 0) return fp16(w), within half an fp16 ulp.
    Returns the largest ratio error / bound seen.
    """
    q, s16, z16 = o.quantize_int(w, bits, group)
    wdq = o.dequant_int(q, s16, z16, group)
    n, k = w.shape
    err = np.abs(wdq.astype(np.float64) - w.astype(np.float64)).reshape(n, k // group, group)
    s = s16.astype(np.float64)[..., None]
    half_ulp32 = np.spacing(np.abs(wdq)).astype(np.float64).reshape(err.shape) / 2
    half_ulp16 = np.spacing(np.abs(w).astype(np.float16)).astype(np.float64).reshape(err.shape) / 2
    bound = np.where(s > 0, s / 2 + half_ulp32, half_ulp16 + half_ulp32)
    ratio = float((err / bound).max())
    assert ratio <= 1.0, f"round trip exceeds s/2: ratio {ratio}"
    # every non-constant group uses both end codes
    qg = q.reshape(err.shape)
    live = s16 > 0
    assert (qg.min(axis=2)[live] == 0).all(), "a group lacks code 0"
    assert (qg.max(axis=2)[live] == (1 << bits) - 1).all(), "a group lacks code qmax"
    return ratio


def check_roundtrip_nf4(o, w, group=64):
    """|w' - w| <= a * (max half gap of the codebook, or |v| - 1 past the ends) + 1/2 ulp."""
    cb = o.nf4_codebook().astype(np.float64)
    q, a16 = o.quantize_nf4(w, group)
    wdq = o.dequant_nf4(q, a16, group)
    n, k = w.shape
    a = a16.astype(np.float64)[..., None]
    w64 = w.astype(np.float64).reshape(n, k // group, group)
    v = w64 / a
    halfgap = float(np.max(np.diff(cb))) / 2
    reach = np.maximum(halfgap, np.abs(v) - 1.0)
    bound = a * reach * (1 + 1e-12) + np.spacing(np.abs(wdq)).reshape(v.shape) / 2
    err = np.abs(wdq.astype(np.float64).reshape(v.shape) - w64)
    ratio = float((err / bound).max())
    assert ratio <= 1.0, f"NF4 round trip exceeds bound: {ratio}"
    return ratio


# ---------------------------------------------------------------------------
# P3 / P4: codebook and nearest-code rule
# ---------------------------------------------------------------------------
def check_codebook(o):
    """Invariants of the NormalFloat construction, via an independent inverse CDF.

    Source: Ultra LLM Engine, Core Components > Quantization, ``nf4`` row
    (QLoRA codebook).  Checked against scipy's normal quantile function (a
    different implementation from the oracle's) and against the defining
    property: the positive entries, scaled back, sit at equally spaced
    normal-CDF probabilities from 0.5 to p*, the negative ones likewise.
    """
    from scipy.stats import norm
    c = o.nf4_codebook()
    assert c.dtype == np.float32 and c.shape == (16,)
    assert (np.diff(c) > 0).all(), "not strictly increasing"
    assert c[0] == -1.0 and c[7] == 0.0 and c[15] == 1.0
    assert (c < 0).sum() == 7 and (c > 0).sum() == 8
    p = o.NF4_PSTAR
    top = norm.ppf(p)
    pos = norm.ppf(np.linspace(p, 0.5, 9)[:-1])
    neg = -norm.ppf(np.linspace(p, 0.5, 8)[:-1])
    ref = (np.sort(np.concatenate([pos, [0.0], neg])) / top).astype(np.float32)
    assert np.array_equal(ref.view(np.uint32), c.view(np.uint32)), "scipy route differs"
    probs_pos = norm.cdf(c[8:].astype(np.float64) * top)
    assert np.allclose(probs_pos, np.linspace(0.5, p, 9)[1:], atol=1e-6)
    probs_neg = norm.cdf(-c[:7].astype(np.float64) * top)
    assert np.allclose(np.sort(probs_neg), np.linspace(0.5, p, 8)[1:], atol=1e-6)


def check_nearest_bruteforce(o, seed=0, n=16, k=256):
    """NF4 codes equal a brute-force argmin over |v - C_j| (first index on ties)."""
    c = o.nf4_codebook().astype(np.float64)
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    # plant exact midpoint ties where the midpoint is an fp32 value: between 0
    # and C[8] the midpoint is C[8]/2; force a = 1 by placing 1.0 in the group
    w[0, 0] = 1.0
    w[0, 1] = np.float32(c[8] / 2)     # midway between C[7] = 0 and C[8]
    w[0, 2] = np.float32(c[6] / 2)     # midway between C[6] and C[7] = 0
    q, a16 = o.quantize_nf4(w, 64)
    v = w.astype(np.float64).reshape(n, k // 64, 64) / a16.astype(np.float64)[..., None]
    d = np.abs(v[..., None] - c)
    brute = d.argmin(axis=-1).reshape(n, k)    # argmin returns the first minimum
    assert np.array_equal(q, brute.astype(np.uint8))
    assert q[0, 1] == 7 and q[0, 2] == 6, "a tie must go to the lower index"


# ---------------------------------------------------------------------------
# P5 / P6: products
# ---------------------------------------------------------------------------
def check_products_exact(o, seed=0, m=3, n=5, k=48):
    """fp64 products agree with exact rational dot products on tiny shapes.

    Bound for an fp64 dot product of length k: k * 2^-53 * sum |x*w|.
    Shapes are non-square so a transposed operand cannot pass.
    """
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k)).astype(np.float16)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    for ref_fn, xs, ws in ((o.gemv_ref, x.astype(np.float64), w.astype(np.float64)),
                           (o.gemm_ref, o.bf16_rne(x.astype(np.float32)).astype(np.float64),
                            o.bf16_rne(w).astype(np.float64))):
        y = ref_fn(x, w)
        assert y.shape == (m, n)
        for i in range(m):
            for j in range(n):
                exact = sum(Fraction(float(xs[i, t])) * Fraction(float(ws[j, t])) for t in range(k))
                mag = float(np.abs(xs[i] * ws[j]).sum())
                assert abs(Fraction(float(y[i, j])) - exact) <= Fraction(k * mag) * Fraction(2) ** -53


def check_one_hot(o, seed=0, n=7, k=64):
    """x = e_t returns column t of w' (GEMV) and of bf16(w') (GEMM) exactly."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    eye = np.eye(k, dtype=np.float16)
    assert np.array_equal(o.gemv_ref(eye, w), w.astype(np.float64).T)
    assert np.array_equal(o.gemm_ref(eye, w), o.bf16_rne(w).astype(np.float64).T)


def check_int8_integer_matmul(o, seed=0, m=4, n=6, k=128, group=64):
    """INT8 with s = 1, z = 0 (integer weights spanning 0..255) is an integer matmul."""
    rng = np.random.default_rng(seed)
    wi = rng.integers(0, 256, size=(n, k))
    wi[:, ::group] = 0
    wi[:, 1::group] = 255
    x = rng.integers(-8, 9, size=(m, k)).astype(np.float16)
    codes, params = o.quantize_pack(wi.astype(np.float32), "int8", group)
    assert np.array_equal(codes, wi.astype(np.uint8))
    wdq = o.dequant_packed(codes, params, "int8", group, k)
    y = o.gemv_ref(x, wdq)
    assert np.array_equal(y, (x.astype(np.int64) @ wi.T).astype(np.float64))


def check_bf16(o, seed=0):
    """bf16 rounding equals torch's CPU conversion (nearest, ties to even)."""
    import torch
    rng = np.random.default_rng(seed)
    a = (rng.standard_normal(4096) * 10.0 ** rng.integers(-6, 6, 4096)).astype(np.float32)
    ties = rng.integers(0, 2 ** 31, 512, dtype=np.uint64).astype(np.uint32)
    ties = (ties & np.uint32(0x7F7F0000)) | np.uint32(0x8000)      # exact halfway cases
    a = np.concatenate([a, ties.view(np.float32), -ties.view(np.float32)])
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(o.bf16_rne(a).view(np.uint32), ref.view(np.uint32))
    # hand values: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1.0);
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6 -> even (1 + 2^-6)
    hv = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    assert o.bf16_rne(hv).tolist() == [1.0, 1 + 2 ** -6, 1 + 2 ** -7]


def check_fp16_conversion(seed=0):
    """numpy's fp32 -> fp16 conversion (the oracle's primitive) rounds to nearest even."""
    import torch
    rng = np.random.default_rng(seed)
    a = (rng.standard_normal(8192) * 10.0 ** rng.integers(-9, 5, 8192)).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.float16).numpy()
    assert np.array_equal(a.astype(np.float16).view(np.uint16), ref.view(np.uint16))
    # hand values: 1 + 2^-11 is halfway -> 1.0; 1 + 3*2^-11 -> 1 + 2^-9
    hv = np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 2 ** -4], dtype=np.float32)
    assert hv.astype(np.float16).view(np.uint16).tolist() == [0x3C00, 0x3C02, 0x2C00]


# ---------------------------------------------------------------------------
# RMSNorm + RoPE (oracle/norm_rope.py): closed forms and brute force
# ---------------------------------------------------------------------------
COS1, SIN1 = 0.5403023058681398, 0.8414709848078965      # cos 1, sin 1 (radians)
COS2, SIN2 = -0.4161468365471424, 0.9092974268256817     # cos 2, sin 2


def check_rope_table(o):
    """Row 0 is the identity; known angles give the textbook cosines and sines."""
    cos, sin = o.rope_table(10000.0, 8, 201)
    assert cos.shape == (201, 4) and cos.dtype == np.float32 and sin.dtype == np.float32
    assert (cos[0] == 1).all() and (sin[0] == 0).all()
    # pair 0 turns by p radians; pair 2 of 4 (d = 8) by p / 100
    assert cos[1, 0] == np.float32(COS1) and sin[1, 0] == np.float32(SIN1)
    assert cos[100, 2] == np.float32(COS1) and sin[100, 2] == np.float32(SIN1)
    assert cos[200, 2] == np.float32(COS2) and sin[200, 2] == np.float32(SIN2)
    assert cos[2, 0] == np.float32(COS2) and sin[2, 0] == np.float32(SIN2)
    unit = cos.astype(np.float64) ** 2 + sin.astype(np.float64) ** 2
    assert np.abs(unit - 1).max() <= 2.0 ** -22


def check_rmsnorm_identity(o, seed=0):
    """At position 0 the rotation is the identity, so y is the RMSNorm alone."""
    rng = np.random.default_rng(seed)
    d = 16
    cos, sin = o.rope_table(10000.0, d, 4)
    x = rng.standard_normal((5, 3, d)).astype(np.float16)
    pos = np.zeros(5, dtype=np.int64)
    y = o.rmsnorm_rope(x, np.ones(d, np.float32), pos, cos, sin, 0.0)
    assert np.abs(np.sqrt(np.mean(y * y, axis=-1)) - 1).max() <= 1e-12
    y2 = o.rmsnorm_rope((x.astype(np.float32) * 2).astype(np.float16), np.ones(d, np.float32), pos, cos, sin, 0.0)
    assert np.abs(y2 - y).max() <= 1e-12                       # scale invariance
    eps = np.float32(0.25)
    ye = o.rmsnorm_rope(x, np.ones(d, np.float32), pos, cos, sin, eps)
    xf = x.astype(np.float64)
    ms = np.mean(xf * xf, axis=-1)
    want = np.sqrt(ms / (ms + np.float64(eps)))                # rms of the output, closed form
    assert np.abs(np.sqrt(np.mean(ye * ye, axis=-1)) - want).max() <= 1e-12
    g = rng.uniform(0.5, 1.5, d).astype(np.float32)
    yg = o.rmsnorm_rope(x, g, pos, cos, sin, 0.0)
    assert np.abs(yg - y * g.astype(np.float64)).max() <= 1e-12


def check_rope_pair_norms(o, seed=1):
    """(a c - b s)^2 + (b c + a s)^2 = (a^2 + b^2)(c^2 + s^2) for every pair (i, i + D/2)."""
    rng = np.random.default_rng(seed)
    d, h = 32, 16
    cos, sin = o.rope_table(10000.0, d, 512)
    x = rng.standard_normal((7, 4, d)).astype(np.float16)
    g = rng.uniform(0.5, 1.5, d).astype(np.float32)
    pos = rng.integers(0, 512, 7)
    y = o.rmsnorm_rope(x, g, pos, cos, sin, 1e-5)
    u = o.rmsnorm_rope(x, g, np.zeros(7, dtype=np.int64), cos, sin, 1e-5)
    c = cos[pos].astype(np.float64)[:, None, :]
    s = sin[pos].astype(np.float64)[:, None, :]
    lhs = y[..., :h] ** 2 + y[..., h:] ** 2
    rhs = (u[..., :h] ** 2 + u[..., h:] ** 2) * (c * c + s * s)
    assert np.abs(lhs - rhs).max() <= 1e-12 * rhs.max()


def check_rope_composition(o, seed=2):
    """Turning by p1 and then by p2 equals turning by p1 + p2 (angle addition)."""
    rng = np.random.default_rng(seed)
    d = 16
    cos, sin = o.rope_table(10000.0, d, 300)
    x = rng.standard_normal((6, 2, d)).astype(np.float16)
    one = np.ones(d, np.float32)
    p1, p2 = rng.integers(0, 150, 6), rng.integers(0, 150, 6)
    y1 = o.rmsnorm_rope(x, one, p1, cos, sin, 0.0)              # rms 1 afterwards
    y12 = o.rmsnorm_rope(y1, one, p2, cos, sin, 0.0)
    y3 = o.rmsnorm_rope(x, one, p1 + p2, cos, sin, 0.0)
    assert np.abs(y12 - y3).max() <= 2e-6                      # fp32 table entries


def check_rope_bruteforce(o, seed=3):
    """Scalar loops with explicit 2x2 rotations from math.cos / math.sin."""
    import math
    rng = np.random.default_rng(seed)
    d, h, theta, eps = 6, 3, 10000.0, 1e-3
    cos, sin = o.rope_table(theta, d, 64)
    x = rng.standard_normal((4, 2, d)).astype(np.float16)
    g = rng.uniform(0.5, 1.5, d).astype(np.float32)
    pos = rng.integers(0, 64, 4)
    y = o.rmsnorm_rope(x, g, pos, cos, sin, eps)
    for t in range(4):
        for hh in range(2):
            v = [float(a) for a in x[t, hh]]
            r = 1.0 / math.sqrt(sum(a * a for a in v) / d + float(np.float32(eps)))
            u = [v[i] * r * float(g[i]) for i in range(d)]
            for i in range(h):
                ang = float(pos[t]) * theta ** (-2.0 * i / d)
                c, s = math.cos(ang), math.sin(ang)
                ya = u[i] * c - u[i + h] * s
                yb = u[i + h] * c + u[i] * s
                assert abs(y[t, hh, i] - ya) <= 1e-6 and abs(y[t, hh, i + h] - yb) <= 1e-6, (t, hh, i)


# ---------------------------------------------------------------------------
# Dynamic activation quantization and the integer-dot GEMV (R-AQ, R-AD)
# ---------------------------------------------------------------------------
def check_a8_grid(o, group=32, m=3, groups=4, seed=4):
    """Groups built on the grid j * 2^e with a +-127 * 2^e element: the codes are
    j exactly and s_x = 2^e; points halfway between grid values round to even."""
    rng = np.random.default_rng(seed)
    k = group * groups
    x = np.zeros((m, k), dtype=np.float64)
    want_q = np.zeros((m, k), dtype=np.int64)
    want_s = np.zeros((m, groups), dtype=np.float64)
    for i in range(m):
        for g in range(groups):
            e = int(rng.integers(-10, 4))
            j = rng.integers(-126, 127, size=group)
            j[0] = 127 if rng.random() < 0.5 else -127
            half = np.zeros(group)
            half[1:5] = 0.5                         # (j + 0.5) * 2^e: a tie for rint
            j[1:5] = rng.integers(-100, 100, size=4)
            x[i, g * group:(g + 1) * group] = (j + half) * 2.0 ** e
            rounded = j + np.where(half > 0, np.where(j % 2 == 0, 0, 1), 0)  # ties to even
            want_q[i, g * group:(g + 1) * group] = rounded
            want_s[i, g] = 2.0 ** e
    x16 = x.astype(np.float16)
    assert np.array_equal(x16.astype(np.float64), x), "grid values must be exact in fp16"
    q, s_x = o.quantize_activations(x16, group)
    assert q.dtype == np.int8
    assert np.array_equal(q.astype(np.int64), want_q)
    assert np.array_equal(s_x.astype(np.float64), want_s)


def check_a8_roundtrip(o, group=64, seed=5):
    """|x - s_x q| <= s_x / 2 (plus fp32 slop); each group's largest |x| maps to +-127;
    codes stay in [-127, 127]; an all-zero group gives codes 0 and scale 0."""
    rng = np.random.default_rng(seed)
    m, k = 4, group * 6
    x = (rng.standard_normal((m, k)) * rng.choice([1e-3, 1.0, 300.0], size=(m, 1))).astype(np.float16)
    x[1, group:2 * group] = 0
    q, s_x = o.quantize_activations(x, group)
    qg = q.astype(np.int64).reshape(m, k // group, group)
    xg = x.astype(np.float64).reshape(m, k // group, group)
    sx = s_x.astype(np.float64)[..., None]
    assert (np.abs(qg) <= 127).all()
    assert (np.abs(xg - sx * qg) <= sx * (0.5 + 2.0 ** -18)).all()
    top = np.abs(xg).argmax(axis=-1)
    hit = np.take_along_axis(np.abs(qg), top[..., None], axis=-1)[..., 0]
    nz = np.abs(xg).max(axis=-1) > 0
    assert (hit[nz] == 127).all()
    assert (qg[1, 1] == 0).all() and s_x[1, 1] == 0


def check_a8_products(o, seed=6):
    """The grouped integer form equals the plain dot product of the dequantized
    activations and weights (both fp64), on non-square shapes."""
    rng = np.random.default_rng(seed)
    for bits, group in ((2, 16), (4, 64), (8, 128)):
        m, n, k = 3, 5, group * 5
        x = (rng.standard_normal((m, k)) * 2.0).astype(np.float16)
        w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
        q_w, s16, z16 = o.quantize_int(w, bits, group)
        q_x, s_x = o.quantize_activations(x, group)
        y = o.gemv_a8_ref(q_x, s_x, q_w, s16, z16, group)
        xd = o.dequant_activations(q_x, s_x, group)
        wd = (q_w.astype(np.float64).reshape(n, k // group, group) * s16.astype(np.float64)[..., None]
              + z16.astype(np.float64)[..., None]).reshape(n, k)
        want = xd @ wd.T
        assert y.shape == (m, n)
        assert np.allclose(y, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def check_a8_bruteforce(o, seed=7):
    """Element-by-element loops on a tiny case (m=2, n=3, k=64, G=16)."""
    rng = np.random.default_rng(seed)
    m, n, k, group = 2, 3, 64, 16
    x = (rng.standard_normal((m, k)) * 3.0).astype(np.float16)
    w = (rng.standard_normal((n, k)) * 0.05).astype(np.float32)
    q_w, s16, z16 = o.quantize_int(w, 4, group)
    q_x, s_x = o.quantize_activations(x, group)
    y = o.gemv_a8_ref(q_x, s_x, q_w, s16, z16, group)
    for i in range(m):
        for j in range(n):
            acc = 0.0
            for t in range(k):
                g = t // group
                xv = float(s_x[i, g]) * int(q_x[i, t])
                wv = int(q_w[j, t]) * float(s16[j, g]) + float(z16[j, g])
                acc += xv * wv
            assert abs(acc - y[i, j]) <= 1e-12 * max(1.0, abs(acc))


# ---------------------------------------------------------------------------
# GGUF Q4_0 / Q8_0 blocks (readings R-GG, R-GI)
# ---------------------------------------------------------------------------
_GGUF_TYPES = {"q4_0": 2, "q8_0": 8}


def load_gguf_cases():
    """Parse tests/golden/gguf_blocks_handbuilt.txt into a list of case dicts."""
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "gguf_blocks_handbuilt.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("case "):
                _, name, fmt, n, k = line.split()
                cur = dict(name=name, gtype=_GGUF_TYPES[fmt], n=int(n[2:]), k=int(k[2:]),
                           blocks={}, values={})
                cases.append(cur)
                continue
            key, val = line.split(":", 1)
            m = re.fullmatch(r"(blocks|values)(\d+)", key)
            kind, row = m.group(1), int(m.group(2))
            if kind == "blocks":
                cur["blocks"][row] = bytes(int(b, 16) for b in val.split())
            else:
                vals = []
                for tok in val.split():
                    rep = re.fullmatch(r"(.+)\{(\d+)\}", tok)
                    v, c = (rep.group(1), int(rep.group(2))) if rep else (tok, 1)
                    vals += [Fraction(v)] * c
                cur["values"][row] = vals
    return cases


def _gguf_blob(case):
    return np.frombuffer(b"".join(case["blocks"][r] for r in range(case["n"])), dtype=np.uint8)


def check_gguf_golden(o):
    """Decode each hand-built block row; every value must equal the fixture.

    Source: the Q4_0 / Q8_0 formats the Ultra LLM Engine page names (Roadmap
    Ideas), laid out as the public GGUF definition (R-GG); the expected values
    are derived by hand in the fixture file."""
    for case in load_gguf_cases():
        w = o.decode_gguf(_gguf_blob(case), case["gtype"], case["n"], case["k"])
        assert w.shape == (case["n"], case["k"]), case["name"]
        for r in range(case["n"]):
            want = [float(v) for v in case["values"][r]]
            assert len(want) == case["k"], case["name"]
            assert w[r].tolist() == want, (case["name"], r)


def check_gguf_placement(o):
    """Brute force over positions: one marked value per block lands where the
    format puts it, and blocks and rows land in order (distinct d per block)."""
    one = np.float16(1.0).view(np.uint16)
    for p in range(32):
        b = np.zeros(18, dtype=np.uint8)
        b[0], b[1] = one & 0xFF, one >> 8
        b[2:] = 0x88                                            # every nibble 8 -> 0
        j = p % 16
        b[2 + j] = 0x89 if p < 16 else 0x98                     # this value -> 1
        w = o.decode_gguf(b, 2, 1, 32)[0]
        assert w[p] == 1.0 and np.count_nonzero(w) == 1, ("q4_0", p)
        b8 = np.zeros(34, dtype=np.uint8)
        b8[0], b8[1] = one & 0xFF, one >> 8
        b8[2 + p] = 1
        w8 = o.decode_gguf(b8, 8, 1, 32)[0]
        assert w8[p] == 1.0 and np.count_nonzero(w8) == 1, ("q8_0", p)
    n, nb = 3, 4
    for gtype, size, fill in ((2, 18, 0x99), (8, 34, 0x01)):   # every value 1 * d
        blob = np.full((n, nb, size), fill, dtype=np.uint8)
        ds = np.arange(1, n * nb + 1, dtype=np.float16).reshape(n, nb)
        bits = ds.view(np.uint16)
        blob[..., 0], blob[..., 1] = bits & 0xFF, bits >> 8
        w = o.decode_gguf(blob.reshape(-1), gtype, n, nb * 32)
        want = np.repeat(ds.astype(np.float64), 32, axis=1)
        assert np.array_equal(w, want), gtype


def check_gguf_q8_identity(o, seed=8):
    """Q8_0 with d = 1 gives the signed bytes; d = 2^e scales them exactly."""
    rng = np.random.default_rng(seed)
    n, k = 4, 256
    q = rng.integers(-128, 128, size=(n, k // 32, 32)).astype(np.int8)
    for e in (0, -7, 5):
        d = np.float16(2.0 ** e).view(np.uint16)
        blob = np.zeros((n, k // 32, 34), dtype=np.uint8)
        blob[..., 0], blob[..., 1] = d & 0xFF, d >> 8
        blob[..., 2:] = q.view(np.uint8)
        w = o.decode_gguf(blob.reshape(-1), 8, n, k)
        assert np.array_equal(w, q.reshape(n, k).astype(np.float64) * 2.0 ** e), e


def random_gguf(gtype, n, k, seed, dmax=0.05):
    """Random blocks from the shared seeded generator (uniform bytes, fp16 d)."""
    return workloads.make_gguf_blocks(gtype, n, k, seed=seed, dmax=dmax)


def check_gguf_int_form(o, seed=9):
    """The INT form (R-GI) dequantizes to the decoded blocks, value for value,
    and refuses scales whose zero point leaves fp16 or that are not finite."""
    for gtype in (2, 8):
        n, k = 5, 320
        blob = random_gguf(gtype, n, k, seed + gtype)
        q, s16, z16 = o.gguf_as_int(blob, gtype, n, k)
        assert q.dtype == np.uint8 and s16.shape == (n, k // 32) and z16.shape == (n, k // 32)
        wd = o.dequant_int(q, s16, z16, 32)
        assert np.array_equal(wd.astype(np.float64), o.decode_gguf(blob, gtype, n, k)), gtype
    # largest scales that still fit, and the first that do not
    for gtype, ok, bad in ((2, 8188.0, 8192.0), (8, 511.75, 512.0)):
        size = 18 if gtype == 2 else 34
        for d, fits in ((ok, True), (bad, False), (np.inf, False), (np.nan, False)):
            b = np.full(size, 0x5A, dtype=np.uint8)
            bits = np.float16(d).view(np.uint16)
            b[0], b[1] = bits & 0xFF, bits >> 8
            if fits:
                q, s16, z16 = o.gguf_as_int(b, gtype, 1, 32)
                assert np.array_equal(o.dequant_int(q, s16, z16, 32).astype(np.float64),
                                      o.decode_gguf(b, gtype, 1, 32)), (gtype, d)
            else:
                try:
                    o.gguf_as_int(b, gtype, 1, 32)
                except ValueError:
                    continue
                raise AssertionError(f"scale {d} accepted for type {gtype}")
