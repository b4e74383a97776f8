"""GPU parity of the activation-quantized GEMV (uq_gemv_a8) and its quantizer.

The int8 activation codes and scales must match the oracle bit for bit (both
sides take the fp32 decisions of reading R-AQ); the products must pass the
gate against the oracle's grouped integer form (reading R-AD), and in fact sit
within fp32 rounding of it.
"""
import numpy as np
import pytest

import oracle as o
import workloads
from tests.gpu_util import Guarded, dev, gate, note, packed_on_device

pytestmark = pytest.mark.gpu

INT_LAYOUTS = [("int2", g) for g in (16, 32, 64, 128)] + [("int4", g) for g in (32, 64, 128)] + \
              [("int8", g) for g in (32, 64, 128)]
BITS = {"int2": 2, "int4": 4, "int8": 8}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU (gfx950)"
    yield
    torch.cuda.synchronize()


def quantize_on_gpu(lib, x, group):
    import torch
    m, k = x.shape
    q = torch.full((m * k + 64,), 0x55, dtype=torch.int8, device="cuda:0")
    sx = Guarded(m * (k // group))
    lib.uq_quantize_activations(group, dev(x), q.data_ptr(), sx.ptr, m, k)
    torch.cuda.synchronize()
    qh = q.cpu().numpy()
    assert (qh[m * k:] == 0x55).all(), "write past the codes"
    return qh[:m * k].reshape(m, k), sx.result().reshape(m, k // group)


def a8_ref(w, x, scheme, group):
    q_w, s16, z16 = o.quantize_int(w, BITS[scheme], group)
    q_x, s_x = o.quantize_activations(x, group)
    y = o.gemv_a8_ref(q_x, s_x, q_w, s16, z16, group)
    xd = o.dequant_activations(q_x, s_x, group)
    wd = o.dequant_int(q_w, s16, z16, group)
    return y, xd, wd


def run_a8(lib, lay, codes, params, x, m):
    y = Guarded(m * lay.n)
    lib.uq_gemv_a8(lay, codes, params, dev(x[:m]), y.ptr, m)
    return y.result().reshape(m, lay.n)


def tight(y, ref, label):
    """fp32 scaling of exact integer sums: far inside the gate."""
    err = np.linalg.norm(np.asarray(y, np.float64) - ref) / max(np.linalg.norm(ref), 1e-300)
    assert err <= 2e-6, f"{label}: rel-L2 {err:.2e} beyond fp32 rounding"


@pytest.mark.parametrize("group", [16, 32, 64, 128])
def test_quantizer_bit_exact(lib, group):
    rng = np.random.default_rng(40 + group)
    m, k = 5, group * 24
    x = (rng.standard_normal((m, k)) * rng.choice([1e-4, 0.3, 7.0, 2000.0], size=(m, 1))).astype(np.float16)
    x[2, :group] = 0                                            # an all-zero group
    x[3, group:2 * group] = np.float16(-3.5)                    # a constant group
    # ties: (j + 1/2) * 2^e next to a +-127 * 2^e element
    e = -3
    j = rng.integers(-100, 100, size=group)
    tie = ((j + 0.5) * 2.0 ** e).astype(np.float16)
    tie[0] = np.float16(127 * 2.0 ** e)
    x[4, 2 * group:3 * group] = tie
    note(f"a8 quantize G{group}")
    q, sx = quantize_on_gpu(lib, x, group)
    q_ref, sx_ref = o.quantize_activations(x, group)
    assert np.array_equal(q, q_ref)
    assert np.array_equal(sx.view(np.uint32), sx_ref.view(np.uint32))


@pytest.mark.parametrize("scheme,group", INT_LAYOUTS)
def test_gemv_a8_parity(lib, scheme, group):
    for n, k, seed in ((37, 4 * max(group, 128 // BITS[scheme] * 2), 41), (300, 2048, 42)):
        w, x = workloads.make_random(n, k, 8, seed=seed, outliers=True)
        lay, codes, params = packed_on_device(lib, scheme, group, w)
        y_ref, xd, wd = a8_ref(w, x, scheme, group)
        for m in (1, 2, 3, 5, 8):
            note(f"a8 gemv {scheme} G{group} n={n} k={k} m={m}")
            y = run_a8(lib, lay, codes, params, x, m)
            gate(y, y_ref[:m], xd[:m], wd, f"a8 {scheme} G{group} {n}x{k} m={m}")
            tight(y, y_ref[:m], f"a8 {scheme} G{group} {n}x{k} m={m}")


def test_gemv_a8_long_k(lib):
    """K past one staged block for every M (several K blocks)."""
    n, k = 70, 40960
    w, x = workloads.make_random(n, k, 8, seed=43, outliers=True)
    for scheme, group in (("int4", 64), ("int2", 16), ("int8", 128)):
        lay, codes, params = packed_on_device(lib, scheme, group, w)
        y_ref, xd, wd = a8_ref(w, x, scheme, group)
        for m in (1, 8):
            note(f"a8 long k {scheme} G{group} m={m}")
            y = run_a8(lib, lay, codes, params, x, m)
            gate(y, y_ref[:m], xd[:m], wd, f"a8 long k {scheme} m={m}")
            tight(y, y_ref[:m], f"a8 long k {scheme} m={m}")


def test_gemv_a8_batched_equivalence(lib):
    """Row i of an M-row call equals the single-row call: bit for bit where both
    run the dot-product kernel (INT2 G32, INT2 G16 at 2 rows, and K in one
    block), within fp32 rounding where 2-8 rows run on the integer matrix cores
    (INT4 / INT8; INT2 G16 from 3 rows), whose rows agree bit for bit across M."""
    n, k = 200, 2048
    w, x = workloads.make_random(n, k, 8, seed=44, outliers=True)
    for scheme, group in (("int4", 64), ("int2", 32), ("int8", 64), ("int8", 128), ("int4", 32), ("int8", 32),
                          ("int2", 16)):
        lay, codes, params = packed_on_device(lib, scheme, group, w)
        ys = [run_a8(lib, lay, codes, params, x[i:i + 1], 1)[0] for i in range(8)]
        full = {}
        for m in (2, 3, 4, 8):
            note(f"a8 batched equivalence {scheme} G{group} m={m}")
            y = run_a8(lib, lay, codes, params, x, m)
            full[m] = y
            if (scheme, group) == ("int2", 32) or ((scheme, group) == ("int2", 16) and m == 2):
                for i in range(m):
                    assert np.array_equal(y[i], ys[i]), (scheme, group, m, i)
            else:
                tight(y, np.stack(ys[:m]).astype(np.float64), f"a8 equiv {scheme} G{group} m={m}")
        if (scheme, group) != ("int2", 32):
            # one kernel per set of row counts (INT2 G16: the dot product at two
            # rows, the matrix cores from three)
            sets = ((3, 4, 8),) if (scheme, group) == ("int2", 16) else ((2, 3, 4, 8),)
            for ms in sets:
                for m in ms[:-1]:
                    assert np.array_equal(full[m].view(np.uint32), full[ms[-1]][:m].view(np.uint32)), (scheme, group, m)


def test_gemv_a8_zero_activations(lib):
    n, k = 50, 1024
    w, _ = workloads.make_random(n, k, 1, seed=45, outliers=True)
    lay, codes, params = packed_on_device(lib, "int4", 64, w)
    x = np.zeros((8, k), dtype=np.float16)
    note("a8 zero activations")
    assert (run_a8(lib, lay, codes, params, x, 8) == 0).all()


@pytest.mark.parametrize("name,ms", [("int4_g64_k4096_n11008", (1, 4)), ("int8_g128_k4096_n4096", (1, 8)),
                                     ("int2_g16_k4096_n4096", (1, 8))])
def test_gemv_a8_full_workloads(lib, name, ms):
    wl = workloads.WORKLOADS[name]
    w, x = workloads.make_workload(wl)
    lay, codes, params = packed_on_device(lib, wl.scheme, wl.group, w)
    y_ref, xd, wd = a8_ref(w, x[:max(ms)], wl.scheme, wl.group)
    for m in ms:
        note(f"a8 full workload {name} m={m}")
        y = run_a8(lib, lay, codes, params, x, m)
        gate(y, y_ref[:m], xd[:m], wd, f"a8 {name} m={m}")
        tight(y, y_ref[:m], f"a8 {name} m={m}")


@pytest.mark.parametrize("name,ms", [("q4_0_k4096_n11008", (1, 2, 4)), ("q8_0_k4096_n4096", (1, 8))])
def test_gemv_a8_full_gguf_workloads(lib, name, ms):
    """GGUF Q4_0 / Q8_0 blocks through the import, then the A8 GEMV at full size:
    the oracle's reference takes the same blocks as INT codes with (d, -offset*d)."""
    wl = workloads.WORKLOADS[name]
    blob, x = workloads.make_gguf_workload(wl)
    lay, codes, params = lib.uq_import_gguf(wl.gguf, blob, wl.n, wl.k)
    codes, params = dev(codes), dev(params)
    q_w, s16, z16 = o.gguf_as_int(blob, wl.gguf, wl.n, wl.k)
    q_x, s_x = o.quantize_activations(x[:max(ms)], wl.group)
    y_ref = o.gemv_a8_ref(q_x, s_x, q_w, s16, z16, wl.group)
    xd = o.dequant_activations(q_x, s_x, wl.group)
    wd = o.decode_gguf(blob, wl.gguf, wl.n, wl.k)
    for m in ms:
        note(f"a8 full GGUF workload {name} m={m}")
        y = run_a8(lib, lay, codes, params, x, m)
        gate(y, y_ref[:m], xd[:m], wd, f"a8 {name} m={m}")
        tight(y, y_ref[:m], f"a8 {name} m={m}")


def test_gemv_a8_refuses_nf4(lib):
    n, k = 16, 256
    w, x = workloads.make_random(n, k, 1, seed=46)
    lay, codes, params = packed_on_device(lib, "nf4", 64, w)
    with pytest.raises(lib.UQError):
        run_a8(lib, lay, codes, params, x, 1)
