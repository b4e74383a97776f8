"""GPU parity of GGUF Q4_0 / Q8_0 weights imported into the INT layout.

The import re-lays the blocks on the host (INT4 / INT8 with G = 32); the
dequant kernel must then return every block value exactly (as a number), and
the GEMV, GEMM and activation-quantized GEMV must pass the gate against the
oracle's products of the decoded blocks.
"""
import numpy as np
import pytest

import oracle as o
import workloads
from tests.gpu_util import Guarded, dev, gate, note, product

pytestmark = pytest.mark.gpu

TYPES = [("q4_0", 2), ("q8_0", 8)]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU (gfx950)"
    yield
    torch.cuda.synchronize()


def imported(lib, t, n, k, seed, dmax=0.01):
    rng = np.random.default_rng(seed)
    blob = workloads.make_gguf_blocks(t, n, k, dmax=dmax, rng=rng)
    x = workloads.make_x(130, k, rng)
    lay, codes, params = lib.uq_import_gguf(t, blob, n, k)
    wdq = o.decode_gguf(blob, t, n, k).astype(np.float32)
    return blob, x, lay, dev(codes), dev(params), wdq


def run(lib, fn, lay, codes, params, x, m):
    y = Guarded(m * lay.n)
    product(lib, fn, lay, codes, params, dev(x[:m]), y.ptr, m)
    return y.result().reshape(m, lay.n)


@pytest.mark.parametrize("fmt,t", TYPES)
def test_gguf_dequant_exact(lib, fmt, t):
    for n, k, seed in ((37, 256, 60), (130, 2048, 61), (5, 4096, 62)):
        _, _, lay, codes, params, wdq = imported(lib, t, n, k, seed)
        note(f"gguf dequant {fmt} n={n} k={k}")
        out = Guarded(n * k)
        lib.uq_dequant(lay, codes, params, out.ptr)
        assert np.array_equal(out.result().reshape(n, k), wdq), (fmt, n, k)


@pytest.mark.parametrize("fmt,t", TYPES)
def test_gguf_products(lib, fmt, t):
    for n, k, seed in ((37, 256, 63), (300, 2048, 64)):
        blob, x, lay, codes, params, wdq = imported(lib, t, n, k, seed)
        for m in (1, 2, 3, 5, 8):
            note(f"gguf gemv {fmt} n={n} k={k} m={m}")
            gate(run(lib, "uq_gemv", lay, codes, params, x, m), o.gemv_ref(x[:m], wdq), x[:m], wdq,
                 f"gguf gemv {fmt} {n}x{k} m={m}")
        for m in (16, 130):
            note(f"gguf gemm {fmt} n={n} k={k} m={m}")
            xb = o.bf16_rne(x[:m].astype(np.float32))
            gate(run(lib, "uq_gemm", lay, codes, params, x, m), o.gemm_ref(x[:m], wdq), xb, o.bf16_rne(wdq),
                 f"gguf gemm {fmt} {n}x{k} m={m}")
        q_w, s16, z16 = o.gguf_as_int(blob, t, n, k)
        q_x, s_x = o.quantize_activations(x[:8], 32)
        y_ref = o.gemv_a8_ref(q_x, s_x, q_w, s16, z16, 32)
        xd = o.dequant_activations(q_x, s_x, 32)
        for m in (1, 8):
            note(f"gguf gemv_a8 {fmt} n={n} k={k} m={m}")
            y = run(lib, "uq_gemv_a8", lay, codes, params, x, m)
            gate(y, y_ref[:m], xd[:m], wdq, f"gguf a8 {fmt} {n}x{k} m={m}")
            err = np.linalg.norm(y - y_ref[:m]) / np.linalg.norm(y_ref[:m])
            assert err <= 2e-6, f"gguf a8 {fmt} m={m}: rel-L2 {err:.2e} beyond fp32 rounding"


@pytest.mark.parametrize("fmt,t", TYPES)
def test_gguf_extreme_scales(lib, fmt, t):
    """Largest accepted scales, subnormal and zero scales in one matrix."""
    n, k = 24, 512
    blob, x, _, _, _, _ = imported(lib, t, n, k, 65)
    size = workloads.GGUF_BLOCK_BYTES[t]
    top = 8188.0 if t == 2 else 511.75
    d = np.resize(np.array([top, -top, 2.0 ** -24, 0.0, -0.0, 1e-3, -3e-2, 0.5], dtype=np.float16),
                  n * (k // 32))
    b = blob.reshape(-1, size)
    bits = d.view(np.uint16)
    b[:, 0], b[:, 1] = bits & 0xFF, bits >> 8
    blob = b.reshape(-1)
    lay, codes, params = lib.uq_import_gguf(t, blob, n, k)
    codes, params = dev(codes), dev(params)
    wdq = o.decode_gguf(blob, t, n, k).astype(np.float32)
    note(f"gguf extreme scales {fmt} dequant")
    out = Guarded(n * k)
    lib.uq_dequant(lay, codes, params, out.ptr)
    assert np.array_equal(out.result().reshape(n, k), wdq)
    xs = (x * np.float16(0.01)).astype(np.float16)      # keep y within fp32 comfortably
    for fn, m in (("uq_gemv", 1), ("uq_gemv", 8), ("uq_gemm", 16)):
        note(f"gguf extreme scales {fmt} {fn} m={m}")
        y = run(lib, fn, lay, codes, params, xs, m)
        if fn == "uq_gemm":
            gate(y, o.gemm_ref(xs[:m], wdq), o.bf16_rne(xs[:m].astype(np.float32)), o.bf16_rne(wdq), fn)
        else:
            gate(y, o.gemv_ref(xs[:m], wdq), xs[:m], wdq, fn)
