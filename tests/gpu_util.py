"""Helpers for the GPU parity tests: device buffers, guard bands, and the gate."""
from __future__ import annotations

import sys

import numpy as np

import oracle as o
import workloads

REL_L2_MAX = 1e-3
ABS_COEF = 2e-3
GUARD = 64          # fp32 guard elements on each side of an output (256 B keeps 16-byte alignment)
SENTINEL = np.float32(-1.2345678e30)


def note(msg: str) -> None:
    """Name the case about to run on the GPU (flushed, so it survives a crash)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev(arr: np.ndarray):
    """Copy a host array to cuda:0 (uint16 data travels as int16: same bits)."""
    import torch
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        arr = arr.view(np.int16)
    return torch.from_numpy(arr).to("cuda:0")


class Guarded:
    """An fp32 output of `count` elements with sentinel guard bands on both sides."""

    def __init__(self, count: int):
        import torch
        self.count = count
        self.buf = torch.full((count + 2 * GUARD,), float(SENTINEL), dtype=torch.float32, device="cuda:0")

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr() + GUARD * 4

    def result(self) -> np.ndarray:
        import torch
        torch.cuda.synchronize()
        h = self.buf.cpu().numpy()
        assert (h[:GUARD] == SENTINEL).all(), "write before the output"
        assert (h[GUARD + self.count:] == SENTINEL).all(), "write past the output"
        out = h[GUARD:GUARD + self.count]
        assert not (out == SENTINEL).any(), "output element left unwritten"
        return out


def product(lib, fn, lay, codes, params, x, y, m, stream=None):
    """Call uq_gemv / uq_gemm / uq_gemv_a8; uq_gemm gets a fresh zero-filled workspace."""
    if fn == "uq_gemm":
        lib.uq_gemm(lay, codes, params, x, y, m, lib.gemm_workspace(lay, m), stream=stream)
    else:
        getattr(lib, fn)(lay, codes, params, x, y, m, stream=stream)


def packed_on_device(lib, scheme, group, w):
    """Pack with the library's host packer and copy to the GPU."""
    lay = lib.layout(scheme, group, w.shape[0], w.shape[1])
    codes, params = lib.uq_pack_weights(lay, w)
    return lay, dev(codes), dev(params)


def workload_on_device(lib, wl):
    """(layout, codes and params on the GPU, the oracle's w' fp32 [n, k], x) of a
    workload: fp32 weights through the packer, or GGUF blocks through the import."""
    if wl.gguf:
        blob, x = workloads.make_gguf_workload(wl)
        lay, codes, params = lib.uq_import_gguf(wl.gguf, blob, wl.n, wl.k)
        wdq = o.decode_gguf(blob, wl.gguf, wl.n, wl.k).astype(np.float32)
        return lay, dev(codes), dev(params), wdq, x
    w, x = workloads.make_workload(wl)
    lay, codes, params = packed_on_device(lib, wl.scheme, wl.group, w)
    return lay, codes, params, oracle_dequant(w, wl.scheme, wl.group), x


def oracle_dequant(w, scheme, group):
    codes, params = o.quantize_pack(w, scheme, group)
    return o.dequant_packed(codes, params, scheme, group, w.shape[1])


def gate(y, yref, xs, wdq, label=""):
    """rel-L2 <= 1e-3 and max |y - yref| <= 2e-3 * sqrt(K) * max|x| * max|w'|."""
    y = np.asarray(y, dtype=np.float64)
    yref = np.asarray(yref, dtype=np.float64)
    assert y.shape == yref.shape, (y.shape, yref.shape)
    assert np.isfinite(y).all(), f"{label}: non-finite output"
    k = wdq.shape[1]
    err = y - yref
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(yref), 1e-300))
    maxabs = float(np.abs(err).max()) if err.size else 0.0
    bound = ABS_COEF * np.sqrt(k) * float(np.abs(xs).max()) * float(np.abs(wdq).max())
    assert rel <= REL_L2_MAX, f"{label}: rel-L2 {rel:.3e} > {REL_L2_MAX}"
    assert maxabs <= bound, f"{label}: max abs {maxabs:.3e} > {bound:.3e}"
    return rel, maxabs
