"""GPU edge cases through the C ABI against the oracle (MI355X only).

Degenerate weights (constant groups, all-zero rows), zero and extreme
activations, a single weight row, and the largest M the GEMM serves.  Same
bars as the parity tests: dequant bit for bit, products within the gate.
"""
import numpy as np
import pytest

import oracle as o
import workloads
from tests.gpu_util import Guarded, dev, gate, note, oracle_dequant, packed_on_device, product

pytestmark = pytest.mark.gpu

LAYOUTS = [("int2", 16), ("int4", 64), ("int4", 128), ("int8", 128), ("nf4", 64)]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU (gfx950)"
    yield
    torch.cuda.synchronize()


def run(lib, fn, lay, codes, params, x, m):
    y = Guarded(m * lay.n)
    product(lib, fn, lay, codes, params, dev(x[:m]), y.ptr, m)
    return y.result().reshape(m, lay.n)


def dequant_on_gpu(lib, lay, codes, params):
    w = Guarded(lay.n * lay.k)
    lib.uq_dequant(lay, codes, params, w.ptr)
    return w.result().reshape(lay.n, lay.k)


def check_products(lib, lay, codes, params, x, wdq, label, gemv_ms=(1, 8), gemm_ms=(16, 130)):
    for m in gemv_ms:
        note(f"{label} gemv m={m}")
        gate(run(lib, "uq_gemv", lay, codes, params, x, m), o.gemv_ref(x[:m], wdq), x[:m], wdq, f"{label} gemv m={m}")
    for m in gemm_ms:
        note(f"{label} gemm m={m}")
        xb = o.bf16_rne(x[:m].astype(np.float32))
        gate(run(lib, "uq_gemm", lay, codes, params, x, m), o.gemm_ref(x[:m], wdq), xb, o.bf16_rne(wdq),
             f"{label} gemm m={m}")


@pytest.mark.parametrize("scheme,group", LAYOUTS)
def test_zero_activations_give_zero(lib, scheme, group):
    n, k = 70, 1024
    w, _ = workloads.make_random(n, k, 1, seed=31, outliers=True)
    lay, codes, params = packed_on_device(lib, scheme, group, w)
    x = np.zeros((130, k), dtype=np.float16)
    for fn, m in (("uq_gemv", 1), ("uq_gemv", 8), ("uq_gemm", 16), ("uq_gemm", 130)):
        note(f"zero x {scheme} G{group} {fn} m={m}")
        y = run(lib, fn, lay, codes, params, x, m)
        assert (y == 0).all(), (scheme, group, fn, m)


@pytest.mark.parametrize("scheme,group", LAYOUTS)
def test_constant_groups_and_zero_rows(lib, scheme, group):
    """Groups whose weights are all equal (zero spread: s = 0, or absmax = |c|) and all-zero rows."""
    n, k = 40, 1024
    rng = np.random.default_rng(32)
    w, x = workloads.make_random(n, k, 130, seed=33, outliers=True)
    consts = rng.normal(0.0, 0.05, size=(n, k // group)).astype(np.float32)
    consts[::7] = 0.0
    flat = np.repeat(consts, group, axis=1)
    pick = rng.random((n, k // group)) < 0.5            # half the groups constant
    w = np.where(np.repeat(pick, group, axis=1), flat, w).astype(np.float32)
    w[3] = 0.0                                          # an all-zero row
    w[11] = 0.125                                       # a constant row
    lay, codes, params = packed_on_device(lib, scheme, group, w)
    wdq = oracle_dequant(w, scheme, group)
    note(f"constant groups {scheme} G{group} dequant")
    got = dequant_on_gpu(lib, lay, codes, params)
    assert np.array_equal(got.view(np.uint32), wdq.astype(np.float32).view(np.uint32))
    check_products(lib, lay, codes, params, x, wdq, f"constant groups {scheme} G{group}")


@pytest.mark.parametrize("scheme,group", LAYOUTS)
def test_single_weight_row(lib, scheme, group):
    n, k = 1, 2048
    w, x = workloads.make_random(n, k, 300, seed=34, outliers=True)
    lay, codes, params = packed_on_device(lib, scheme, group, w)
    wdq = oracle_dequant(w, scheme, group)
    check_products(lib, lay, codes, params, x, wdq, f"n=1 {scheme} G{group}", gemm_ms=(16, 300))


@pytest.mark.parametrize("scale", [300.0, 3000.0])
@pytest.mark.parametrize("scheme,group", [("int4", 64), ("int2", 16), ("int8", 128), ("nf4", 64)])
def test_large_activations(lib, scheme, group, scale):
    """Activation outliers of hundreds to thousands (and a few near the fp16 limit)."""
    n, k = 96, 2048
    w, x = workloads.make_random(n, k, 130, seed=35, outliers=True)
    rng = np.random.default_rng(36)
    xs = x.astype(np.float32) * scale
    hot = rng.random(xs.shape) < 0.002
    xs[hot] = np.sign(xs[hot] + 0.5) * 60000.0
    x = np.clip(xs, -65504, 65504).astype(np.float16)
    lay, codes, params = packed_on_device(lib, scheme, group, w)
    wdq = oracle_dequant(w, scheme, group)
    check_products(lib, lay, codes, params, x, wdq, f"x*{scale:g} {scheme} G{group}")


def test_gemm_largest_m(lib):
    """M = 65536 (the most uq_gemm serves): 512 row tiles, every output checked."""
    m, n, k = 65536, 70, 64
    w, x = workloads.make_random(n, k, m, seed=37, outliers=True)
    lay, codes, params = packed_on_device(lib, "int4", 32, w)
    wdq = oracle_dequant(w, "int4", 32)
    note(f"gemm m={m} n={n} k={k}")
    y = run(lib, "uq_gemm", lay, codes, params, x, m)
    xb = o.bf16_rne(x.astype(np.float32))
    gate(y, o.gemm_ref(x, wdq), xb, o.bf16_rne(wdq), "gemm m=65536")


@pytest.mark.parametrize("scheme,group", [("int2", 16), ("int2", 64), ("int4", 32), ("int4", 64), ("int4", 128),
                                          ("int8", 128), ("nf4", 64)])
def test_small_and_mixed_activations(lib, scheme, group):
    """Activations far below 1 (x * 1e-3, 1e-4, 2e-5: fp16 values whose
    division by a code class would fall into fp16 subnormals), activation rows
    of very different sizes in one call (normal, tiny, largest fp16), through
    the single-row and multi-row GEMVs and the GEMM, against the oracle."""
    n, k = 300, 2048
    w, x = workloads.make_random(n, k, 16, seed=51, outliers=True)
    lay, codes, params = packed_on_device(lib, scheme, group, w)
    wdq = oracle_dequant(w, scheme, group)
    xf = x.astype(np.float32)
    for scale in (1e-3, 1e-4, 2e-5):
        xs = (xf * np.float32(scale)).astype(np.float16)
        for m in (1, 2, 8):
            note(f"small x {scheme} G{group} scale={scale} m={m}")
            gate(run(lib, "uq_gemv", lay, codes, params, xs, m), o.gemv_ref(xs[:m], wdq), xs[:m], wdq,
                 f"{scheme} G{group} x*{scale} m={m}")
    mixed = xf.copy()
    mixed[1] *= 1e-4
    mixed[3] *= 2e-5
    mixed[5] = np.clip(mixed[5] * 2e4, -65504, 65504)
    mixed = mixed.astype(np.float16)
    for m in (2, 4, 8):
        note(f"mixed rows {scheme} G{group} m={m}")
        y = run(lib, "uq_gemv", lay, codes, params, mixed, m)
        ref = o.gemv_ref(mixed[:m], wdq)
        for i in range(m):  # each row on its own scale
            gate(y[i:i + 1], ref[i:i + 1], mixed[i:i + 1], wdq, f"{scheme} G{group} mixed m={m} row {i}")
    note(f"small x gemm {scheme} G{group}")
    xs = (xf * np.float32(1e-4)).astype(np.float16)
    xb = o.bf16_rne(xs[:16].astype(np.float32))
    gate(run(lib, "uq_gemm", lay, codes, params, xs, 16), o.gemm_ref(xs[:16], wdq), xb, o.bf16_rne(wdq),
         f"{scheme} G{group} small x gemm")
