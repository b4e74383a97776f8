"""GPU parity of the fused RMSNorm + RoPE kernel against the oracle (MI355X only).

Every output value must lie within one fp16 spacing of the exact (fp64)
result, plus fp32 rounding at the vector's scale (oracle.within_gate); guard
bands around the output must stay untouched.
"""
import numpy as np
import pytest

import oracle as o
import workloads
from tests.gpu_util import note

pytestmark = pytest.mark.gpu
GUARD = 64  # fp16 values of sentinel on each side of the output
SENTINEL = np.int16(0x7E5A)  # a NaN pattern the kernel never writes


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU (gfx950)"
    yield
    torch.cuda.synchronize()


def to_dev(a):
    import torch
    if a.dtype == np.float16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run(lib, x, gamma, pos, cos, sin, eps, in_place=False):
    import torch
    t, h, d = x.shape
    n = t * h * d
    buf = torch.full((n + 2 * GUARD + 8,), int(SENTINEL), dtype=torch.int16, device="cuda")
    y = buf[GUARD:GUARD + n]  # 128-byte offset: 16-byte aligned
    xd = to_dev(x)
    if in_place:
        y.copy_(xd.reshape(-1))
        xd = y
    lib.uq_rmsnorm_rope(xd, y, to_dev(gamma), to_dev(pos.astype(np.int32)), to_dev(cos), to_dev(sin),
                        t, h, d, cos.shape[0], eps)
    torch.cuda.synchronize()
    out = buf.cpu().numpy()
    assert (out[:GUARD] == SENTINEL).all() and (out[GUARD + n:] == SENTINEL).all(), "guard band written"
    return out[GUARD:GUARD + n].view(np.float16).reshape(t, h, d)


def check(y, ref, label):
    ok = o.within_gate(y, ref)
    assert ok.all(), f"{label}: {int((~ok).sum())} values outside the gate"


@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_parity_shapes(lib, d):
    rng = np.random.default_rng(d)
    cos, sin = o.rope_table(10000.0, d, 2048)
    for t, h, eps in ((1, 1, 1e-6), (5, 3, 1e-6), (33, 8, 0.5), (130, 2, 1e-5)):
        note(f"rmsnorm_rope d={d} t={t} h={h} eps={eps}")
        x = rng.standard_normal((t, h, d)).astype(np.float16)
        g = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
        pos = rng.integers(0, 2048, t)
        pos[0], pos[-1] = 0, 2047
        y = run(lib, x, g, pos, cos, sin, eps)
        check(y, o.rmsnorm_rope(x, g, pos, cos, sin, eps), f"d={d} t={t} h={h}")


def test_in_place(lib):
    rng = np.random.default_rng(5)
    cos, sin = o.rope_table(500000.0, 128, 512)
    x = rng.standard_normal((17, 4, 128)).astype(np.float16)
    g = (1 + 0.1 * rng.standard_normal(128)).astype(np.float32)
    pos = rng.integers(0, 512, 17)
    note("rmsnorm_rope in place")
    y = run(lib, x, g, pos, cos, sin, 1e-6, in_place=True)
    check(y, o.rmsnorm_rope(x, g, pos, cos, sin, 1e-6), "in place")


def test_value_range(lib):
    """Large and tiny magnitudes, and an all-zero vector (eps > 0 keeps it zero)."""
    rng = np.random.default_rng(6)
    cos, sin = o.rope_table(10000.0, 256, 64)
    x = (rng.standard_normal((6, 2, 256)) * np.array([3e4, 1.0, 1e-3, 1e-5, 1.0, 1.0])[:, None, None])
    x = np.clip(x, -65504, 65504).astype(np.float16)
    x[4] = 0
    g = (1 + 0.1 * rng.standard_normal(256)).astype(np.float32)
    pos = rng.integers(0, 64, 6)
    note("rmsnorm_rope value range")
    y = run(lib, x, g, pos, cos, sin, 1e-6)
    ref = o.rmsnorm_rope(x, g, pos, cos, sin, 1e-6)
    check(y, ref, "value range")
    assert (y[4] == 0).all()


def test_out_of_range_positions_give_nan(lib):
    rng = np.random.default_rng(7)
    cos, sin = o.rope_table(10000.0, 64, 100)
    x = rng.standard_normal((6, 3, 64)).astype(np.float16)
    g = np.ones(64, np.float32)
    pos = np.array([0, -1, 99, 100, 5, 2**31 - 1])
    note("rmsnorm_rope positions out of range")
    y = run(lib, x, g, pos, cos, sin, 1e-6)
    bad = np.array([False, True, False, True, False, True])
    assert np.isnan(y[bad].astype(np.float32)).all()
    good = ~bad
    check(y[good], o.rmsnorm_rope(x[good], g, pos[good], cos, sin, 1e-6), "in-range tokens")


@pytest.mark.parametrize("name", list(workloads.NORM_ROPE))
def test_full_workload(lib, name):
    wl = workloads.NORM_ROPE[name]
    x, g, pos = workloads.make_norm_rope(wl)
    cos, sin = o.rope_table(wl.theta, wl.head_dim, wl.max_pos)
    note(f"rmsnorm_rope full {name}")
    y = run(lib, x, g, pos, cos, sin, wl.eps)
    check(y, o.rmsnorm_rope(x, g, pos, cos, sin, wl.eps), name)
