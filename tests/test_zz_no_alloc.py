"""uq_gemm_noalloc (the GEMM in the library's fixed per-GPU scratch, for
callers that cannot allocate) against uq_gemm with its own workspace, through
the C ABI.  Several calls in a row on one stream, each smaller than the one
before where it matters: the scratch keeps the previous call's contents, so
this checks that nothing a call reads is left over from an earlier one."""
import numpy as np
import pytest

import oracle as o
import workloads
from tests.gpu_util import Guarded, dev, gate, note, oracle_dequant, packed_on_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU (gfx950)"
    yield
    torch.cuda.synchronize()


def _both(lib, lay, codes, params, x, m):
    y_na = Guarded(m * lay.n)
    lib.uq_gemm_noalloc(lay, codes, params, dev(x[:m]), y_na.ptr, m)
    got = y_na.result().reshape(m, lay.n)
    y_ws = Guarded(m * lay.n)
    lib.uq_gemm(lay, codes, params, dev(x[:m]), y_ws.ptr, m, lib.gemm_workspace(lay, m))
    return got, y_ws.result().reshape(m, lay.n)


@pytest.mark.parametrize("scheme,group,n,k,ms", [
    ("int4", 128, 700, 2048, (200, 40)),      # bf16 staging, then a K-split call
    ("int4", 64, 384, 1024, (64, 16, 1)),     # K-split calls of shrinking size
    ("int2", 16, 4100, 512, (300, 130)),      # 128-row tiles, then 64-row tiles
    ("nf4", 64, 129, 4096, (33, 17)),
])
def test_noalloc_matches_uq_gemm(lib, scheme, group, n, k, ms):
    w, x = workloads.make_random(n, k, max(ms), seed=41, outliers=True)
    lay, codes, params = packed_on_device(lib, scheme, group, w)
    wdq = oracle_dequant(w, scheme, group)
    for m in ms:
        note(f"noalloc {scheme} G{group} n={n} k={k} m={m}")
        got, want = _both(lib, lay, codes, params, x, m)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (scheme, m)
        xb = o.bf16_rne(x[:m].astype(np.float32))
        gate(got, o.gemm_ref(x[:m], wdq), xb, o.bf16_rne(wdq), f"noalloc {scheme} m={m}")


def test_noalloc_refuses_more_than_its_scratch(lib):
    """A call whose workspace would not fit the fixed scratch is refused before any HIP call."""
    lay = lib.layout("int4", 128, 4096, 4096)
    m = 65536
    assert lib.uq_gemm_workspace_size(lay, m) > lib.GEMM_NOALLOC_MAX_BYTES
    with pytest.raises(lib.UQError) as e:
        lib.uq_gemm_noalloc(lay, 1 << 20, 1 << 20, 1 << 20, 1 << 20, m)
    assert e.value.name == "UQ_ERR_WORKSPACE"
