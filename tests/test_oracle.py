"""Oracle pins (CPU only): the oracle checked against facts outside itself."""
import numpy as np
import pytest

import oracle as o
import workloads
from tests import pins

INT_CASES = [(2, g) for g in (16, 32, 64, 128)] + [(4, g) for g in (32, 64, 128)] + \
            [(8, g) for g in (32, 64, 128)]


def test_fp16_primitive_rounds_to_nearest_even():
    pins.check_fp16_conversion()


def test_bf16_matches_torch_and_hand_values():
    pins.check_bf16(o)


def test_packing_hand_built_golden():
    pins.check_packing_golden(o)


@pytest.mark.parametrize("bits,group", INT_CASES)
def test_grid_recovery(bits, group):
    for seed in range(3):
        pins.check_grid_recovery(o, bits, group, seed=seed)


def test_codebook():
    pins.check_codebook(o)


def test_nearest_code_bruteforce():
    for seed in range(4):
        pins.check_nearest_bruteforce(o, seed=seed)


@pytest.mark.parametrize("k", [16, 32, 48, 64])
def test_products_against_exact_rationals(k):
    pins.check_products_exact(o, seed=k, k=k)


def test_one_hot():
    pins.check_one_hot(o)


def test_int8_unit_scale_is_integer_matmul():
    pins.check_int8_integer_matmul(o)


def test_constant_and_zero_groups():
    """Constant INT groups: s = 0, all codes 0, w' = fp16(w).  All-zero NF4 group: code 7, w' = 0."""
    w = np.full((2, 64), 0.3, dtype=np.float32)
    w[1, :32] = -1.25
    q, s16, z16 = o.quantize_int(w, 4, 32)
    assert (q == 0).all() and (s16 == 0).all()
    assert np.array_equal(o.dequant_int(q, s16, z16, 32), w.astype(np.float16).astype(np.float32))
    z = np.zeros((1, 64), dtype=np.float32)
    qn, a16 = o.quantize_nf4(z, 64)
    assert (qn == 7).all() and (a16 == 0).all()
    assert (o.dequant_nf4(qn, a16) == 0).all()


def test_pack_unpack_roundtrip():
    rng = np.random.default_rng(1)
    for bits in (2, 4, 8):
        q = rng.integers(0, 1 << bits, size=(5, 128)).astype(np.uint8)
        assert np.array_equal(o.unpack_codes(o.pack_codes(q, bits), bits, 128), q)


@pytest.mark.parametrize("name", ["int4_g32_k256_n768", "int8_g128_k4096_n4096",
                                  "int2_g16_k4096_n4096"])
def test_roundtrip_bound_configs(name):
    wl = workloads.WORKLOADS[name]
    w, _ = workloads.make_workload(wl)
    ratio = pins.check_roundtrip_int(o, w, o.BITS[wl.scheme], wl.group)
    assert ratio <= 1.0


@pytest.mark.slow
def test_roundtrip_bound_int4_outliers_full():
    wl = workloads.WORKLOADS["int4_g64_k4096_n11008"]
    w, _ = workloads.make_workload(wl)
    pins.check_roundtrip_int(o, w, 4, 64)
    wg = workloads.WORKLOADS["int4_g128_k4096_n11008_gemm"]
    w2, _ = workloads.make_workload(wg)
    pins.check_roundtrip_int(o, w2, 4, 128)


@pytest.mark.slow
def test_roundtrip_bound_nf4_full():
    wl = workloads.WORKLOADS["nf4_g64_k4096_n14336"]
    w, _ = workloads.make_workload(wl)
    pins.check_roundtrip_nf4(o, w, 64)


def test_roundtrip_nf4_small():
    w, _ = workloads.make_random(64, 512, 1, seed=3, outliers=True)
    pins.check_roundtrip_nf4(o, w, 64)


# ---------------------------------------------------------------------------
# RMSNorm + RoPE
# ---------------------------------------------------------------------------
def test_rope_table():
    pins.check_rope_table(o)


def test_rmsnorm_identity():
    pins.check_rmsnorm_identity(o)


def test_rope_pair_norms():
    pins.check_rope_pair_norms(o)


def test_rope_composition():
    pins.check_rope_composition(o)


def test_rope_bruteforce():
    pins.check_rope_bruteforce(o)


def test_fp16_spacing():
    import torch
    v = np.array([1.0, 1.5, 2.0, 3.0e-3, 1.0e-6, 60000.0, 6.1e-5])
    t = torch.tensor(v, dtype=torch.float16)
    nxt = torch.nextafter(t, torch.tensor(np.inf, dtype=torch.float16)).double().numpy()
    assert np.array_equal(o.fp16_spacing(v), nxt - t.double().numpy())


def test_norm_rope_gate():
    """The gate accepts the fp16 rounding of the exact result and rejects a
    one-spacing-plus error on an ordinary value."""
    rng = np.random.default_rng(4)
    cos, sin = o.rope_table(10000.0, 64, 128)
    x = rng.standard_normal((9, 2, 64)).astype(np.float16)
    ref = o.rmsnorm_rope(x, np.ones(64, np.float32), rng.integers(0, 128, 9), cos, sin, 1e-6)
    assert o.within_gate(ref.astype(np.float16), ref).all()
    bad = ref.astype(np.float16).astype(np.float64)
    i = np.unravel_index(np.argmax(np.abs(ref)), ref.shape)
    bad[i] += 3 * o.fp16_spacing(ref[i])
    assert not o.within_gate(bad, ref).all()


# Dynamic activation quantization and the integer-dot GEMV (R-AQ, R-AD)
def test_a8_grid():
    pins.check_a8_grid(o)


def test_a8_roundtrip():
    pins.check_a8_roundtrip(o)


def test_a8_products():
    pins.check_a8_products(o)


def test_a8_bruteforce():
    pins.check_a8_bruteforce(o)


def test_gguf_golden():
    pins.check_gguf_golden(o)


def test_gguf_placement():
    pins.check_gguf_placement(o)


def test_gguf_q8_identity():
    pins.check_gguf_q8_identity(o)


def test_gguf_int_form():
    pins.check_gguf_int_form(o)


def test_gguf_rejects_bad_shapes():
    with pytest.raises(ValueError):
        o.decode_gguf(np.zeros(18, np.uint8), 3, 1, 32)      # not a Q4_0 / Q8_0 type
    with pytest.raises(ValueError):
        o.decode_gguf(np.zeros(18, np.uint8), 2, 1, 48)      # k not whole blocks
    with pytest.raises(ValueError):
        o.decode_gguf(np.zeros(17, np.uint8), 2, 1, 32)      # short blob
