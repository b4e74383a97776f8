"""The host-side C++ of libuq under AddressSanitizer + UndefinedBehaviorSanitizer.

The packer, the GGUF re-layout, the rotary table, the GEMM workspace size and
the argument checks of the device entry points are compiled with g++ (no HIP)
together with tests/sanitize_driver.cpp.  The driver runs them over the
hand-built golden matrices, random and edge-value weights, GGUF blocks with
edge scales and every documented error path; any sanitizer report fails the
test, and the sanitized build's bytes must equal the oracle's.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle as o
from tests import pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gemm_group_wise_amd", "csrc")
SOURCES = ["uq_pack.cpp", "uq_gguf.cpp", "rope_table.cpp", "uq_check.cpp", "uq_host_api.cpp"]
SCHEME_ID = {"int2": 1, "int4": 2, "int8": 3, "nf4": 4}
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("asan") / "sanitize_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-pthread",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "sanitize_driver.cpp")] + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", out]
    p = subprocess.run(cmd, capture_output=True, text=True)
    assert p.returncode == 0, p.stderr[-4000:]
    return out


def run(driver, *args):
    p = subprocess.run([driver, *map(str, args)], capture_output=True, text=True, env=ENV, timeout=600)
    assert "Sanitizer" not in p.stderr and "runtime error" not in p.stderr, p.stderr[-4000:]
    return p.returncode, p.stderr


def test_error_paths_and_checks(driver):
    rc, err = run(driver, "checks")
    assert rc == 0, err


def _pack_case(driver, tmp_path, scheme, group, w):
    n, k = w.shape
    wf, cf, pf = tmp_path / "w.f32", tmp_path / "codes", tmp_path / "params"
    np.ascontiguousarray(w, dtype=np.float32).tofile(wf)
    rc, err = run(driver, "pack", SCHEME_ID[scheme], group, n, k, wf, cf, pf)
    assert rc == 0, (rc, err)
    codes = np.fromfile(cf, dtype=np.uint8).reshape(n, -1)
    params = np.fromfile(pf, dtype=np.uint16)
    rc_, rp = o.quantize_pack(w, scheme, group)
    assert np.array_equal(codes, rc_), (scheme, group)
    assert np.array_equal(params, rp.reshape(-1).view(np.uint16)), (scheme, group)


def test_pack_golden(driver, tmp_path):
    cb = o.nf4_codebook()
    for case in pins.load_packing_cases():
        _pack_case(driver, tmp_path, case["scheme"], case["group"], pins.build_case_weights(case, cb))


@pytest.mark.parametrize("scheme,group", [("int2", 16), ("int2", 128), ("int4", 32), ("int4", 64), ("int4", 128),
                                          ("int8", 32), ("int8", 128), ("nf4", 64)])
def test_pack_edge_values(driver, tmp_path, scheme, group):
    k = 4 * max(group, 128 // o.BITS[scheme])
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((9, k)) * 0.02).astype(np.float32)
    w[0] = 0.0
    w[1] = 0.37
    w[2] = rng.standard_normal(k).astype(np.float32) * 13000.0
    w[2, 0], w[2, 1] = 65504.0, -65504.0
    w[3] = rng.standard_normal(k).astype(np.float32) * 1e-6
    w[4] = np.float32(1e-3) * (np.arange(k) % 7).astype(np.float32)
    w[5, ::2] = -w[5, 1::2]
    cb = o.nf4_codebook()
    w[6] = np.resize(cb, k)
    w[7] = np.resize((cb[:-1] + cb[1:]) / 2, k)
    w[8] = np.float32(6e-8)
    _pack_case(driver, tmp_path, scheme, group, np.clip(w, -65504, 65504).astype(np.float32))


@pytest.mark.parametrize("t,bits", [(2, 4), (8, 8)])
def test_gguf_import(driver, tmp_path, t, bits):
    n, k = 5, 32 * 9
    blob = pins.random_gguf(t, n, k, 9)
    b = blob.reshape(-1, 18 if t == 2 else 34)
    top = 8188.0 if t == 2 else 511.75
    d = np.array([2.0 ** -24, -2.0 ** -24, 0.0, -0.0, top, -top, 6.1e-5, 1.0, -3.0] * n, dtype=np.float16)
    bits16 = d.view(np.uint16)
    b[:, 0], b[:, 1] = bits16 & 0xFF, bits16 >> 8
    bf, cf, pf = tmp_path / "blocks", tmp_path / "codes", tmp_path / "params"
    b.reshape(-1).tofile(bf)
    rc, err = run(driver, "gguf", t, n, k, bf, cf, pf)
    assert rc == 0, (rc, err)
    q, s16, z16 = o.gguf_as_int(b.reshape(-1), t, n, k)
    assert np.array_equal(np.fromfile(cf, dtype=np.uint8), o.pack_codes(q, bits).reshape(-1))
    assert np.array_equal(np.fromfile(pf, dtype=np.uint16), o.pack_params_int(s16, z16).reshape(-1))


@pytest.mark.parametrize("theta,d,p", [(10000.0, 128, 300), (500000.0, 64, 17), (1e6, 6, 5)])
def test_rope_table(driver, tmp_path, theta, d, p):
    cf, sf = tmp_path / "cos", tmp_path / "sin"
    rc, err = run(driver, "rope", theta, d, p, cf, sf)
    assert rc == 0, (rc, err)
    oc, os_ = o.rope_table(theta, d, p)
    for got, want in ((np.fromfile(cf, dtype=np.float32), oc), (np.fromfile(sf, dtype=np.float32), os_)):
        ulps = np.abs(got.view(np.int32).astype(np.int64) - want.reshape(-1).view(np.int32).astype(np.int64))
        assert ulps.max() <= 1
