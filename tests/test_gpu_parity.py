"""GPU parity: the HIP path through the C ABI against the oracle (MI355X only).

Dequantized weights must match bit for bit; products must pass the gate
(rel-L2 <= 1e-3, max abs <= 2e-3 * sqrt(K) * max|x| * max|w'|), and the
one-hot cases must reproduce w' exactly.
"""
import numpy as np
import pytest

import oracle as o
import workloads
from tests.gpu_util import Guarded, dev, gate, note, oracle_dequant, packed_on_device, workload_on_device

pytestmark = pytest.mark.gpu

ALL_LAYOUTS = [("int2", g) for g in (16, 32, 64, 128)] + [("int4", g) for g in (32, 64, 128)] + \
              [("int8", g) for g in (32, 64, 128)] + [("nf4", 64)]
CW = {"int2": 64, "int4": 32, "int8": 16, "nf4": 32}


def small_k(scheme, group, mult=4):
    return mult * max(group, CW[scheme])


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU (gfx950)"
    props = torch.cuda.get_device_properties(0)
    note(f"device: {props.name} {getattr(props, 'gcnArchName', '')}")
    yield
    torch.cuda.synchronize()


def run_gemv(lib, lay, codes, params, x, m):
    y = Guarded(m * lay.n)
    lib.uq_gemv(lay, codes, params, dev(x[:m]), y.ptr, m)
    return y.result().reshape(m, lay.n)


def run_gemm(lib, lay, codes, params, x, m, ws=None):
    y = Guarded(m * lay.n)
    lib.uq_gemm(lay, codes, params, dev(x[:m]), y.ptr, m, lib.gemm_workspace(lay, m) if ws is None else ws)
    return y.result().reshape(m, lay.n)


# ---------------------------------------------------------------------------
# Dequant: bit-exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("scheme,group", ALL_LAYOUTS)
def test_dequant_bit_exact(lib, scheme, group):
    for n, k, seed in ((37, small_k(scheme, group), 0), (5, 4096, 1), (130, small_k(scheme, group, 2), 2)):
        note(f"dequant {scheme} G{group} n={n} k={k}")
        w, _ = workloads.make_random(n, k, 1, seed=seed, outliers=True)
        lay, codes, params = packed_on_device(lib, scheme, group, w)
        out = Guarded(n * k)
        lib.uq_dequant(lay, codes, params, out.ptr)
        got = out.result().reshape(n, k)
        want = oracle_dequant(w, scheme, group)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (scheme, group, n, k)


# ---------------------------------------------------------------------------
# GEMV (M <= 8)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("scheme,group", ALL_LAYOUTS)
def test_gemv_parity_small(lib, scheme, group):
    for n, k, seed in ((37, small_k(scheme, group), 3), (1000, 1024, 4), (17, 4096, 5)):
        w, x = workloads.make_random(n, k, 8, seed=seed, outliers=True)
        lay, codes, params = packed_on_device(lib, scheme, group, w)
        wdq = oracle_dequant(w, scheme, group)
        for m in (1, 2, 3, 4, 5, 8):
            note(f"gemv {scheme} G{group} n={n} k={k} m={m}")
            y = run_gemv(lib, lay, codes, params, x, m)
            gate(y, o.gemv_ref(x[:m], wdq), x[:m], wdq, f"{scheme} G{group} {n}x{k} m={m}")


@pytest.mark.parametrize("scheme,group", [l for l in ALL_LAYOUTS if l[0] != "nf4"])
def test_gemv_one_hot_bit_exact(lib, scheme, group):
    """x = e_k reproduces column k of w' exactly (the scale times an integer code is exact)."""
    n, k = 45, small_k(scheme, group)
    w, _ = workloads.make_random(n, k, 1, seed=6, outliers=True)
    lay, codes, params = packed_on_device(lib, scheme, group, w)
    wdq = oracle_dequant(w, scheme, group)
    cols = [0, 1, k // 2 + 3, k - 1, 5, 17, 31 % k, k - 2]
    x = np.zeros((8, k), dtype=np.float16)
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    for m in (1, 3, 8):
        note(f"gemv one-hot {scheme} G{group} m={m}")
        y = run_gemv(lib, lay, codes, params, x, m)
        want = np.stack([wdq[:, c] for c in cols[:m]])
        assert np.array_equal(y.view(np.uint32), want.view(np.uint32)), (scheme, group, m)


def test_gemv_one_hot_nf4(lib):
    """NF4 products use the codebook as fp16 high + low parts (about 22 bits): x = e_k
    gives w' to within 2^-20 relative (plus 2^-23 of the largest weight for codes near 0)."""
    n, k = 45, 256
    w, _ = workloads.make_random(n, k, 1, seed=7)
    lay, codes, params = packed_on_device(lib, "nf4", 64, w)
    wdq = oracle_dequant(w, "nf4", 64)
    x = np.zeros((4, k), dtype=np.float16)
    cols = [0, 63, 64, 255]
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    note("gemv one-hot nf4")
    y = run_gemv(lib, lay, codes, params, x, 4)
    want = np.stack([wdq[:, c] for c in cols]).astype(np.float64)
    assert (np.abs(y - want) <= np.abs(want) * 2.0 ** -20 + 2.0 ** -23 * np.abs(wdq).max()).all()


def test_gemv_batched_equivalence(lib):
    """Row i of an M-row GEMV equals the single-row GEMV of x[i] within the gate
    (the pages' batched-decode equivalence; not bitwise, since the orders of
    the fp32 sums differ).  INT4 / INT8 calls with 2 to 8 rows (INT2 G16 with
    5 to 8) run on the matrix cores, whose sum order does not depend on M:
    their rows agree bit for bit across M, as do the dot-product kernel's
    rows (INT4 G32 on a matrix of fewer than 8192 rows runs the dot product up
    to 4 rows and the matrix cores from 5).  NF4 keeps the dot-product kernel for every M; with
    K in one LDS block of activations its rows agree with the single-row call
    bit for bit.
    """
    for scheme, group in (("int4", 64), ("int2", 16), ("int8", 128), ("nf4", 64), ("int4", 32), ("int2", 64)):
        for k in (1024, 4096):
            w, x = workloads.make_random(300, k, 8, seed=8, outliers=True)
            lay, codes, params = packed_on_device(lib, scheme, group, w)
            wdq = oracle_dequant(w, scheme, group)
            ys = [run_gemv(lib, lay, codes, params, x[i:i + 1], 1)[0] for i in range(8)]
            full = {}
            for m in (2, 3, 4, 5, 8):
                note(f"gemv batched equivalence {scheme} G{group} k={k} m={m}")
                y = run_gemv(lib, lay, codes, params, x, m)
                full[m] = y
                gate(y, np.stack(ys[:m]).astype(np.float64), x[:m], wdq, f"equiv {scheme} m={m}")
                gate(y, o.gemv_ref(x[:m], wdq), x[:m], wdq, f"oracle {scheme} m={m}")
                if scheme == "nf4" and k == 1024:
                    for i in range(m):
                        assert np.array_equal(y[i], ys[i]), (scheme, group, m, i)
            # calls served by one kernel agree bit for bit across M: INT4 / INT8
            # rows 2-8 (matrix cores), INT2 rows 5-8 (matrix cores, G16) and 2-4
            # (dot product, whose rows do not depend on M either)
            if scheme == "int4" and group == 32:
                sets = ((2, 3, 4), (5, 8))  # 300 rows: the dot product up to 4 rows, the matrix cores from 5
            elif scheme in ("int4", "int8"):
                sets = ((2, 3, 4, 5, 8),)
            elif scheme == "int2":
                sets = ((2, 3, 4), (5, 8)) if group == 16 else ((2, 3, 4, 5, 8),)
            else:
                sets = ()
            for ms in sets:
                for m in ms[:-1]:
                    assert np.array_equal(full[m].view(np.uint32), full[ms[-1]][:m].view(np.uint32)), (scheme, group, k, m)


def test_gemv_g32_large_matrix_rows_agree(lib):
    """INT4 G32 on a matrix of 8192 or more weight rows runs on the matrix cores
    from three activation rows: rows of M = 3, 4, 5, 8 agree bit for bit (one
    kernel, a sum order that does not depend on M) and with the oracle within
    the gate; M = 2 (the dot product) agrees within the gate."""
    w, x = workloads.make_random(8200, 1024, 8, seed=21, outliers=True)
    lay, codes, params = packed_on_device(lib, "int4", 32, w)
    wdq = oracle_dequant(w, "int4", 32)
    full = {}
    for m in (2, 3, 4, 5, 8):
        note(f"gemv int4 G32 n=8200 m={m}")
        full[m] = run_gemv(lib, lay, codes, params, x, m)
        gate(full[m], o.gemv_ref(x[:m], wdq), x[:m], wdq, f"int4 G32 8200 m={m}")
    for m in (3, 4, 5):
        assert np.array_equal(full[m].view(np.uint32), full[8][:m].view(np.uint32)), m


@pytest.mark.parametrize("scheme,group,n,k", [
    ("int4", 64, 300, 4096), ("int4", 128, 777, 4096), ("int4", 64, 11008, 4096), ("int4", 64, 37, 1024),
    ("int4", 128, 129, 2560), ("int4", 64, 100, 16384), ("int8", 32, 333, 1024), ("int8", 64, 45, 2048),
    ("int8", 128, 4096, 4096), ("int8", 128, 61, 8192), ("int8", 32, 17, 3968),
    ("int2", 16, 300, 4096), ("int2", 16, 37, 1024), ("int2", 16, 129, 8192), ("int2", 16, 45, 3584),
    ("int4", 32, 300, 4096), ("int4", 32, 8200, 1024), ("int4", 32, 45, 3584)])
def test_gemv_matrix_core_shapes(lib, scheme, group, n, k):
    """The matrix-core GEMV (2 to 8 activation rows, INT4 groups of 64 / 128 and
    INT8; 5 to 8 rows of INT2 G16 and of INT4 G32, 3 to 8 of INT4 G32 on 8192 or
    more weight rows): one to eight 128-byte blocks per wave, K
    padded up to whole blocks (zero activations, groups past K ignored), a
    ragged last 16-row tile, and 2 / 4 / 8 staged activation rows."""
    w, x = workloads.make_random(n, k, 8, seed=42, outliers=True)
    lay, codes, params = packed_on_device(lib, scheme, group, w)
    wdq = oracle_dequant(w, scheme, group)
    for m in (2, 3, 4, 5, 6, 8):
        note(f"gemv matrix-core {scheme} G{group} n={n} k={k} m={m}")
        y = run_gemv(lib, lay, codes, params, x, m)
        gate(y, o.gemv_ref(x[:m], wdq), x[:m], wdq, f"mfma gemv {scheme} G{group} {n}x{k} m={m}")


@pytest.mark.parametrize("m,k", [(1, 36864), (8, 8192), (4, 8320)])
def test_gemv_k_blocks(lib, m, k):
    """K larger than one LDS block of activations (16384 values over all rows, 32768 for
    INT2), with a ragged last block."""
    w, x = workloads.make_random(70, k, m, seed=9)
    for scheme, group in (("int4", 128), ("int2", 64), ("nf4", 64), ("int8", 64)):
        if k % max(group, CW[scheme]):
            continue
        note(f"gemv k-blocks {scheme} G{group} m={m} k={k}")
        lay, codes, params = packed_on_device(lib, scheme, group, w)
        wdq = oracle_dequant(w, scheme, group)
        y = run_gemv(lib, lay, codes, params, x, m)
        gate(y, o.gemv_ref(x[:m], wdq), x[:m], wdq, f"k-blocks {scheme} m={m} k={k}")


@pytest.mark.parametrize("k", [8192, 8320])
def test_gemv_long_k_many_rows(lib, k):
    """One activation row, K past one block and N large enough for the usual
    rows per wave (INT4 and INT2 then take two rows per wave instead of four),
    a ragged last workgroup (N = 4100) and, at K = 8320, a ragged chunk group."""
    n = 4100
    w, x = workloads.make_random(n, k, 1, seed=90 + k % 7, outliers=True)
    for scheme, group in (("int4", 64), ("int4", 32), ("int4", 128), ("int2", 16), ("int2", 64),
                          ("nf4", 64), ("int8", 128)):
        if k % max(group, CW[scheme]):
            continue
        note(f"gemv long K {scheme} G{group} n={n} k={k} m=1")
        lay, codes, params = packed_on_device(lib, scheme, group, w)
        wdq = oracle_dequant(w, scheme, group)
        y = run_gemv(lib, lay, codes, params, x, 1)
        gate(y, o.gemv_ref(x[:1], wdq), x[:1], wdq, f"long K {scheme} G{group} k={k}")


def test_gemv_on_side_stream(lib):
    import torch
    w, x = workloads.make_random(64, 512, 1, seed=10)
    lay, codes, params = packed_on_device(lib, "int4", 32, w)
    wdq = oracle_dequant(w, "int4", 32)
    s = torch.cuda.Stream()
    xd = dev(x)
    y = Guarded(64)
    torch.cuda.synchronize()
    note("gemv on a side stream")
    lib.uq_gemv(lay, codes, params, xd, y.ptr, 1, stream=s)
    s.synchronize()
    gate(y.result().reshape(1, 64), o.gemv_ref(x, wdq), x, wdq, "side stream")


# ---------------------------------------------------------------------------
# GEMM (bf16 matrix cores)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("scheme,group", ALL_LAYOUTS)
def test_gemm_parity_small(lib, scheme, group):
    for n, k, seed in ((100, 512, 11), (77, small_k(scheme, group), 12)):
        w, x = workloads.make_random(n, k, 130, seed=seed, outliers=True)
        lay, codes, params = packed_on_device(lib, scheme, group, w)
        wdq = oracle_dequant(w, scheme, group)
        for m in (1, 15, 16, 17, 40, 64, 130):
            note(f"gemm {scheme} G{group} n={n} k={k} m={m}")
            y = run_gemm(lib, lay, codes, params, x, m)
            xb = o.bf16_rne(x[:m].astype(np.float32))
            gate(y, o.gemm_ref(x[:m], wdq), xb, o.bf16_rne(wdq), f"gemm {scheme} G{group} m={m}")


@pytest.mark.parametrize("scheme,group", [("int4", 128), ("int2", 16), ("int8", 64), ("nf4", 64)])
def test_gemm_several_row_tiles(lib, scheme, group):
    """M over several row tiles with a partial last one (rows past M are computed, not
    stored), at widths that select each tile height: N = 100 runs 32-row tiles, N = 4100
    64-row tiles and N = 8100 128-row tiles once M > 64 (the grid must reach 128 tiles)."""
    k = 256
    for n, seed in ((100, 21), (4100, 22), (8100, 23)):
        w, x = workloads.make_random(n, k, 513, seed=seed, outliers=True)
        lay, codes, params = packed_on_device(lib, scheme, group, w)
        wdq = oracle_dequant(w, scheme, group)
        for m in (129, 255, 256, 257, 300, 513):
            note(f"gemm row tiles {scheme} G{group} n={n} m={m}")
            y = run_gemm(lib, lay, codes, params, x, m)
            xb = o.bf16_rne(x[:m].astype(np.float32))
            gate(y, o.gemm_ref(x[:m], wdq), xb, o.bf16_rne(wdq), f"gemm {scheme} G{group} n={n} m={m}")


@pytest.mark.parametrize("scheme,group", ALL_LAYOUTS)
def test_gemm_identity_bit_exact(lib, scheme, group):
    """X = I (M = K) returns bf16(w')^T exactly."""
    n, k = 70, 256
    w, _ = workloads.make_random(n, k, 1, seed=13, outliers=True)
    lay, codes, params = packed_on_device(lib, scheme, group, w)
    wdq = oracle_dequant(w, scheme, group)
    x = np.eye(k, dtype=np.float16)
    note(f"gemm identity {scheme} G{group}")
    y = run_gemm(lib, lay, codes, params, x, k)
    want = o.bf16_rne(wdq).T
    assert np.array_equal(y.view(np.uint32), np.ascontiguousarray(want).view(np.uint32))


@pytest.mark.parametrize("k", [96, 160, 224])
def test_gemm_k_tail(lib, k):
    """K not a multiple of the 128-wide K step."""
    w, x = workloads.make_random(65, k, 33, seed=14)
    lay, codes, params = packed_on_device(lib, "int4", 32, w)
    wdq = oracle_dequant(w, "int4", 32)
    note(f"gemm k-tail k={k}")
    y = run_gemm(lib, lay, codes, params, x, 33)
    gate(y, o.gemm_ref(x, wdq), o.bf16_rne(x.astype(np.float32)), o.bf16_rne(wdq), f"k-tail {k}")


def test_gemm_batched_equivalence(lib):
    """Row i of an M-row GEMM equals the single-row GEMM of x[i].

    Up to M = 16 (with K a multiple of 1024) one streaming kernel with 16-row
    tiles serves every M, with one K order and one K split, so rows agree bit
    for bit; above, other tiles cut K differently and rows agree to fp32
    reassociation.  (GEMM and GEMV rows are not compared under the gate: the
    bf16 rounding of w' alone moves the GEMM by ~2e-3 relative to the fp16
    GEMV, which is why the GEMM's oracle applies the same casts.)
    """
    w, x = workloads.make_random(300, 2048, 130, seed=15)
    lay, codes, params = packed_on_device(lib, "int4", 128, w)
    ys = np.stack([run_gemm(lib, lay, codes, params, x[i:i + 1], 1)[0] for i in range(130)])
    for m in (5, 16):
        note(f"gemm batched equivalence m={m}")
        y = run_gemm(lib, lay, codes, params, x, m)
        assert np.array_equal(y.view(np.uint32), ys[:m].view(np.uint32)), m
    for m in (17, 32, 40, 64, 130):
        note(f"gemm batched equivalence m={m}")
        y = run_gemm(lib, lay, codes, params, x, m)
        assert np.abs(y - ys[:m]).max() <= 1e-5 * np.abs(ys[:m]).max(), m


@pytest.mark.parametrize("scheme,group", ALL_LAYOUTS)
def test_gemm_streaming_rows(lib, scheme, group):
    """Up to 32 rows with K a multiple of 256 the GEMM streams codes into
    registers: 16- and 32-row tiles, N with a ragged last tile of 64 weight
    rows; K up to 4096 in blocks of 512 requested at once (K splits with one
    block and with two, and with a split short of a block), other K in
    blocks of 256 with one in flight (K = 1280 and 4864)."""
    for n, k, seed in ((77, 1024, 41), (200, 3072, 42), (2100, 2048, 43), (130, 1280, 44), (70, 4864, 45)):
        w, x = workloads.make_random(n, k, 32, seed=seed, outliers=True)
        lay, codes, params = packed_on_device(lib, scheme, group, w)
        wdq = oracle_dequant(w, scheme, group)
        for m in (1, 7, 16, 17, 31, 32):
            note(f"gemm streaming {scheme} G{group} n={n} k={k} m={m}")
            y = run_gemm(lib, lay, codes, params, x, m)
            xb = o.bf16_rne(x[:m].astype(np.float32))
            gate(y, o.gemm_ref(x[:m], wdq), xb, o.bf16_rne(wdq), f"gemm streaming {scheme} G{group} n={n} k={k} m={m}")
        for m in (16, 32):
            # rows of I: each output is one product, exact through the K split
            note(f"gemm streaming identity {scheme} G{group} n={n} k={k} m={m}")
            e = np.zeros((m, k), dtype=np.float16)
            e[np.arange(m), (np.arange(m) * 37) % k] = 1.0
            y = run_gemm(lib, lay, codes, params, e, m)
            want = o.bf16_rne(wdq).T[(np.arange(m) * 37) % k]
            assert np.array_equal(y.view(np.uint32), np.ascontiguousarray(want).view(np.uint32)), m


@pytest.mark.parametrize("scheme,group", [("int4", 128), ("int2", 16), ("int8", 32), ("nf4", 64), ("int4", 32)])
def test_gemm_k_split(lib, scheme, group):
    """Up to M = 64 the K steps are split over several workgroups and the last
    one to finish a tile adds the partial tiles.  K values give ranges that
    start inside a parameter window, odd step counts and a ragged last tile
    of weight rows; N small enough that every tile is split four ways."""
    for n, k, seed in ((100, 2560, 31), (300, 1536, 32), (129, 4096, 33)):
        w, x = workloads.make_random(n, k, 64, seed=seed, outliers=True)
        lay, codes, params = packed_on_device(lib, scheme, group, w)
        wdq = oracle_dequant(w, scheme, group)
        for m in (1, 16, 33, 64):
            note(f"gemm k split {scheme} G{group} n={n} k={k} m={m}")
            y = run_gemm(lib, lay, codes, params, x, m)
            xb = o.bf16_rne(x[:m].astype(np.float32))
            gate(y, o.gemm_ref(x[:m], wdq), xb, o.bf16_rne(wdq), f"gemm split {scheme} G{group} n={n} k={k} m={m}")


@pytest.mark.parametrize("scheme,group", [("int4", 128), ("int2", 16), ("int8", 64), ("nf4", 64)])
def test_gemm_k_split_identity_bit_exact(lib, scheme, group):
    """X = the first 64 rows of I with K = 2560 (K split over four workgroups):
    each output is one product, so the partial tiles and their sum are exact
    and y = bf16(w')^T[:64] bit for bit."""
    n, k = 70, 2560
    w, _ = workloads.make_random(n, k, 1, seed=34, outliers=True)
    lay, codes, params = packed_on_device(lib, scheme, group, w)
    wdq = oracle_dequant(w, scheme, group)
    x = np.eye(k, dtype=np.float16)[:64]
    note(f"gemm k split identity {scheme} G{group}")
    y = run_gemm(lib, lay, codes, params, x, 64)
    want = o.bf16_rne(wdq).T[:64]
    assert np.array_equal(y.view(np.uint32), np.ascontiguousarray(want).view(np.uint32))


def test_gemm_deterministic(lib):
    """Repeated calls give identical bits (no atomics, fixed summation order)."""
    w, x = workloads.make_random(1000, 4096, 256, seed=16)
    lay, codes, params = packed_on_device(lib, "int4", 128, w)
    for m in (1, 16, 64, 256):
        note(f"gemm deterministic m={m}")
        a = run_gemm(lib, lay, codes, params, x, m)
        b = run_gemm(lib, lay, codes, params, x, m)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), m


def test_gemm_graph_replay(lib):
    """A call captured into a HIP graph on a fresh stream, with no call made
    before the capture, replays the eager result bit for bit, replay after
    replay, with eager work on the same buffers and workspace in between.
    N = 384 makes six tiles, so K is split over two workgroups per tile: the
    replays also check that each call leaves the arrival counters at zero."""
    import torch
    w, x = workloads.make_random(384, 1024, 64, seed=17)
    lay, codes, params = packed_on_device(lib, "int4", 64, w)
    wdq = oracle_dequant(w, "int4", 64)
    xd = dev(x)
    y = torch.empty(64 * 384, dtype=torch.float32, device="cuda")
    ws = lib.gemm_workspace(lay, 64)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    note("gemm graph: capture on a fresh stream")
    with torch.cuda.graph(g, stream=s):
        lib.uq_gemm(lay, codes, params, xd, y, 64, ws, stream=s.cuda_stream)
    want = None
    for r in range(4):
        note(f"gemm graph: replay {r}")
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = y.cpu().numpy().copy()
        if want is None:
            want = run_gemm(lib, lay, codes, params, x, 64)
            gate(want, o.gemm_ref(x, wdq), o.bf16_rne(x.astype(np.float32)), o.bf16_rne(wdq), "graph eager")
        assert np.array_equal(got.view(np.uint32), want.reshape(-1).view(np.uint32)), r
        lib.uq_gemm(lay, codes, params, xd, y, 16, ws)  # eager work in between, same workspace
        torch.cuda.synchronize()


def test_gemm_two_streams(lib):
    """Concurrent calls on two streams, each with its own workspace."""
    import torch
    w, x = workloads.make_random(512, 2048, 200, seed=18)
    lay, codes, params = packed_on_device(lib, "int4", 128, w)
    want_a = run_gemm(lib, lay, codes, params, x, 200)
    want_b = run_gemm(lib, lay, codes, params, x[100:], 100)
    xa, xb = dev(x), dev(x[100:])
    ya = torch.empty(200 * 512, dtype=torch.float32, device="cuda")
    yb = torch.empty(100 * 512, dtype=torch.float32, device="cuda")
    wa, wb = lib.gemm_workspace(lay, 200), lib.gemm_workspace(lay, 100)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    note("gemm two streams")
    for _ in range(3):
        lib.uq_gemm(lay, codes, params, xa, ya, 200, wa, stream=s1.cuda_stream)
        lib.uq_gemm(lay, codes, params, xb, yb, 100, wb, stream=s2.cuda_stream)
    torch.cuda.synchronize()
    assert np.array_equal(ya.cpu().numpy().reshape(200, 512).view(np.uint32), want_a.view(np.uint32))
    assert np.array_equal(yb.cpu().numpy().reshape(100, 512).view(np.uint32), want_b.view(np.uint32))


def test_gemm_workspace_reused_across_sizes(lib):
    """One workspace sized for the largest call serves smaller and split calls in
    turn on one stream (the counters are back at zero after each call)."""
    import torch
    w, x = workloads.make_random(700, 2048, 256, seed=19)
    lay, codes, params = packed_on_device(lib, "int4", 128, w)
    big = max(lib.uq_gemm_workspace_size(lay, m) for m in (1, 16, 64, 256))
    ws = torch.zeros(big, dtype=torch.uint8, device="cuda")
    for m in (64, 1, 256, 16, 64):
        note(f"gemm shared workspace m={m}")
        got = run_gemm(lib, lay, codes, params, x, m, ws=ws)
        want = run_gemm(lib, lay, codes, params, x, m)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), m


# ---------------------------------------------------------------------------
# Full-size workloads, in the launch configuration the benchmark times
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_full_workload(lib, name):
    wl = workloads.WORKLOADS[name]
    lay, codes, params, wdq, x = workload_on_device(lib, wl)
    if wl.path == "gemv":
        note(f"full dequant {name}")
        out = Guarded(wl.n * wl.k)
        lib.uq_dequant(lay, codes, params, out.ptr)
        got = out.result()
        if wl.gguf:   # equal as numbers: the INT form may flip the sign of a zero
            assert np.array_equal(got, wdq.reshape(-1))
        else:
            assert np.array_equal(got.view(np.uint32), wdq.reshape(-1).view(np.uint32))
        del out
    for m in wl.ms:
        note(f"full {wl.path} {name} m={m}")
        if wl.path == "gemv":
            y = run_gemv(lib, lay, codes, params, x, m)
            rel, mx = gate(y, o.gemv_ref(x[:m], wdq), x[:m], wdq, f"{name} m={m}")
        else:
            y = run_gemm(lib, lay, codes, params, x, m)
            rel, mx = gate(y, o.gemm_ref(x[:m], wdq), o.bf16_rne(x[:m].astype(np.float32)),
                           o.bf16_rne(wdq), f"{name} m={m}")
        note(f"  rel-L2 {rel:.3e}  max-abs {mx:.3e}")
