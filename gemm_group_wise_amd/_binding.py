"""ctypes binding of libuq (include/uq.h).  Argument marshalling only.

Device buffers are passed as integers or as torch tensors; streams as
integers or objects with ``cuda_stream``.  When no stream is given the current
torch stream is used.  A tensor is checked before the call (on a GPU,
contiguous, of an accepted dtype and large enough for the layout and m), so a
CPU tensor or a short buffer raises ValueError instead of reaching a kernel;
a plain integer is passed through unchecked (the raw escape hatch).  Every
non-OK status raises :class:`UQError`.  If the library is not built,
importing this module raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libuq.so")

SCHEMES = {"int2": 1, "int4": 2, "int8": 3, "nf4": 4}
BITS = {"int2": 2, "int4": 4, "int8": 8, "nf4": 4}
GGUF_TYPES = {"q4_0": 2, "q8_0": 8}
GGUF_BLOCK_BYTES = {2: 18, 8: 34}
GEMV_MAX_M = 8
GEMM_MAX_M = 65536

STATUS = {0: "UQ_OK", 1: "UQ_ERR_NULL", 2: "UQ_ERR_SHAPE", 3: "UQ_ERR_UNSUPPORTED",
          4: "UQ_ERR_ALIGN", 5: "UQ_ERR_RANGE", 6: "UQ_ERR_HIP", 7: "UQ_ERR_WORKSPACE"}


class UQError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        self.name = STATUS.get(code, f"status {code}")
        super().__init__(f"{fn} failed: {self.name}")


class Layout(ctypes.Structure):
    _fields_ = [("scheme", ctypes.c_int32), ("group", ctypes.c_int32),
                ("n", ctypes.c_int64), ("k", ctypes.c_int64)]

    def __repr__(self):
        return f"Layout(scheme={self.scheme}, group={self.group}, n={self.n}, k={self.k})"


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                      "(or python gemm_group_wise_amd/build.py)")

# torch ships its own HIP runtime, which its libraries load by the unversioned
# name libamdhip64.so.  libuq.so asks for libamdhip64.so.7; if it were opened
# first, the dynamic loader would later map torch's copy as well and the
# process would run two HIP/HSA runtimes on one device.  Importing torch first
# lets libuq.so bind to the runtime torch already loaded (same SONAME).
try:
    import torch  # noqa: F401
except ImportError:  # plain C-ABI use without torch
    torch = None
_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_L = ctypes.POINTER(Layout)
_lib.uq_packed_size.argtypes = [_L, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
_lib.uq_pack_weights.argtypes = [_L, _P, _P, _P]
_lib.uq_import_gguf.argtypes = [ctypes.c_int32, _P, ctypes.c_int64, ctypes.c_int64, _L, _P, _P]
_lib.uq_gemv.argtypes = [_L, _P, _P, _P, _P, ctypes.c_int64, _P]
_lib.uq_gemm.argtypes = [_L, _P, _P, _P, _P, ctypes.c_int64, _P, ctypes.c_size_t, _P]
_lib.uq_gemm_noalloc.argtypes = [_L, _P, _P, _P, _P, ctypes.c_int64, _P]
_lib.uq_probe_read.argtypes = [_P, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32, _P, _P]
_lib.uq_gemm_workspace_size.argtypes = [_L, ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)]
_lib.uq_dequant.argtypes = [_L, _P, _P, _P, _P]
_lib.uq_gemv_a8.argtypes = [_L, _P, _P, _P, _P, ctypes.c_int64, _P]
_lib.uq_quantize_activations.argtypes = [ctypes.c_int32, _P, _P, _P, ctypes.c_int64, ctypes.c_int64, _P]
_lib.uq_nf4_codebook.argtypes = [_P]
_lib.uq_rope_table.argtypes = [ctypes.c_double, ctypes.c_int32, ctypes.c_int64, _P, _P]
_lib.uq_rmsnorm_rope.argtypes = [_P, _P, _P, _P, _P, _P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_int64, ctypes.c_float, _P]
_lib.uq_status_str.argtypes = [ctypes.c_int]
_lib.uq_status_str.restype = ctypes.c_char_p
for _fn in ("uq_packed_size", "uq_pack_weights", "uq_import_gguf", "uq_gemv", "uq_gemm", "uq_dequant",
            "uq_nf4_codebook", "uq_rope_table", "uq_rmsnorm_rope", "uq_gemv_a8", "uq_quantize_activations",
            "uq_gemm_workspace_size", "uq_gemm_noalloc", "uq_probe_read"):
    getattr(_lib, _fn).restype = ctypes.c_int

EXPORTS = ("uq_packed_size", "uq_pack_weights", "uq_import_gguf", "uq_gemv", "uq_gemm", "uq_dequant",
           "uq_nf4_codebook", "uq_rope_table", "uq_rmsnorm_rope", "uq_gemv_a8", "uq_quantize_activations",
           "uq_gemm_workspace_size", "uq_gemm_noalloc", "uq_probe_read", "uq_status_str")
GEMM_NOALLOC_MAX_BYTES = 32 << 20


def _check(fn: str, status: int):
    if status != 0:
        raise UQError(fn, status)


def _ptr(obj, what: str = "buffer", nbytes: int = 0, dtypes: tuple = ()) -> int | None:
    """Device address of `obj`.  An int passes through unchecked; a tensor must
    be on a GPU, contiguous, of one of `dtypes` (names such as "float16"; any
    dtype when empty) and hold at least `nbytes` bytes."""
    if obj is None:
        return None
    if isinstance(obj, int):
        return obj
    if hasattr(obj, "data_ptr"):
        if not getattr(obj, "is_cuda", False):
            raise ValueError(f"{what}: expected a tensor on a GPU, got one on {getattr(obj, 'device', '?')}")
        if dtypes and str(obj.dtype).replace("torch.", "") not in dtypes:
            raise ValueError(f"{what}: dtype {obj.dtype} is not one of {', '.join(dtypes)}")
        if not obj.is_contiguous():
            raise ValueError(f"{what}: tensor is not contiguous")
        have = obj.numel() * obj.element_size()
        if have < nbytes:
            raise ValueError(f"{what}: {have} bytes, the call needs {nbytes}")
        return obj.data_ptr()
    raise TypeError(f"expected a device pointer (int) or a tensor, got {type(obj)!r}")


_U8 = ("uint8", "int8")
_F16 = ("float16", "int16", "uint16")
_F32 = ("float32",)


def _product_ptrs(lay: Layout, codes, params, x, y, m: int):
    """Checked addresses of a product's operands (sizes from the layout and m)."""
    cb, pb = uq_packed_size(lay)
    m = max(int(m), 0)
    return (_ptr(codes, "codes", cb, _U8), _ptr(params, "params", pb, _F16 + ("int32",)),
            _ptr(x, "x", m * lay.k * 2, _F16), _ptr(y, "y", m * lay.n * 4, _F32))


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def layout(scheme: str | int, group: int, n: int, k: int) -> Layout:
    s = SCHEMES[scheme] if isinstance(scheme, str) else int(scheme)
    return Layout(s, group, n, k)


def uq_packed_size(lay: Layout) -> tuple[int, int]:
    cb, pb = ctypes.c_size_t(), ctypes.c_size_t()
    _check("uq_packed_size", _lib.uq_packed_size(ctypes.byref(lay), ctypes.byref(cb), ctypes.byref(pb)))
    return cb.value, pb.value


def uq_pack_weights(lay: Layout, w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Quantize + pack a host fp32 [n, k] matrix; returns (codes uint8, params uint16)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.shape != (lay.n, lay.k):
        raise ValueError(f"w has shape {w.shape}, layout wants {(lay.n, lay.k)}")
    cb, pb = uq_packed_size(lay)
    codes = np.empty((lay.n, cb // lay.n), dtype=np.uint8)
    params = np.empty(pb // 2, dtype=np.uint16)
    _check("uq_pack_weights", _lib.uq_pack_weights(ctypes.byref(lay), w.ctypes.data,
                                                  codes.ctypes.data, params.ctypes.data))
    return codes, params.reshape(lay.n, -1)


def uq_import_gguf(gguf_type: str | int, blocks: np.ndarray, n: int, k: int):
    """Re-lay host GGUF Q4_0 / Q8_0 blocks of an [n, k] matrix; returns
    (layout, codes uint8 [n, -1], params uint16 [n, k / 32, 2])."""
    t = GGUF_TYPES[gguf_type] if isinstance(gguf_type, str) else int(gguf_type)
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(-1)
    shaped = t in GGUF_BLOCK_BYTES and n >= 1 and k >= 32 and k % 32 == 0
    if shaped and blocks.size != n * (k // 32) * GGUF_BLOCK_BYTES[t]:
        # the library cannot see the buffer's length: never let it read past it
        raise ValueError(f"blocks hold {blocks.size} bytes, not {n * (k // 32) * GGUF_BLOCK_BYTES[t]}")
    # buffers for a valid call; on a rejected shape the library writes nothing
    codes = np.empty(n * k // (2 if t == 2 else 1) if shaped else 1, dtype=np.uint8)
    params = np.empty(n * (k // 32) * 2 if shaped else 1, dtype=np.uint16)
    lay = Layout()
    _check("uq_import_gguf", _lib.uq_import_gguf(t, blocks.ctypes.data, int(n), int(k), ctypes.byref(lay),
                                                codes.ctypes.data, params.ctypes.data))
    return lay, codes.reshape(lay.n, -1), params.reshape(lay.n, -1, 2)


def uq_gemv(lay: Layout, codes, params, x, y, m: int, stream=None) -> None:
    _check("uq_gemv", _lib.uq_gemv(ctypes.byref(lay), *_product_ptrs(lay, codes, params, x, y, m),
                                   int(m), _stream(stream)))


def uq_gemm_workspace_size(lay: Layout, m: int) -> int:
    """Bytes of workspace uq_gemm needs for this layout and m (host call)."""
    b = ctypes.c_size_t()
    _check("uq_gemm_workspace_size", _lib.uq_gemm_workspace_size(ctypes.byref(lay), int(m), ctypes.byref(b)))
    return b.value


def gemm_workspace(lay: Layout, m: int, device="cuda"):
    """A zero-filled uint8 device tensor of uq_gemm_workspace_size(lay, m) bytes
    (torch allocates it; the library never does).  Reusable for later calls of
    the same or smaller size on one stream."""
    import torch
    return torch.zeros(max(uq_gemm_workspace_size(lay, m), 1), dtype=torch.uint8, device=device)


def uq_gemm(lay: Layout, codes, params, x, y, m: int, workspace, stream=None) -> None:
    """workspace: a tensor (its size is passed along) or (address, bytes)."""
    if isinstance(workspace, tuple):
        wp, wb = int(workspace[0]), int(workspace[1])
    else:
        wp = _ptr(workspace, "workspace")
        wb = workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else 0
    _check("uq_gemm", _lib.uq_gemm(ctypes.byref(lay), *_product_ptrs(lay, codes, params, x, y, m), int(m),
                                   wp, wb, _stream(stream)))


def uq_gemm_noalloc(lay: Layout, codes, params, x, y, m: int, stream=None) -> None:
    """uq_gemm in the library's fixed per-GPU scratch (no workspace argument;
    calls on one GPU must not overlap)."""
    _check("uq_gemm_noalloc", _lib.uq_gemm_noalloc(ctypes.byref(lay), *_product_ptrs(lay, codes, params, x, y, m),
                                                   int(m), _stream(stream)))


def uq_gemv_a8(lay: Layout, codes, params, x, y, m: int, stream=None) -> None:
    _check("uq_gemv_a8", _lib.uq_gemv_a8(ctypes.byref(lay), *_product_ptrs(lay, codes, params, x, y, m),
                                         int(m), _stream(stream)))


def uq_quantize_activations(group: int, x, q, sx, m: int, k: int, stream=None) -> None:
    mk = max(int(m), 0) * max(int(k), 0)
    groups = max(int(m), 0) * (max(int(k), 0) // int(group)) if int(group) > 0 else 0
    _check("uq_quantize_activations", _lib.uq_quantize_activations(
        int(group), _ptr(x, "x", 2 * mk, _F16), _ptr(q, "q", mk, ("int8",)), _ptr(sx, "sx", 4 * groups, _F32),
        int(m), int(k), _stream(stream)))


def uq_dequant(lay: Layout, codes, params, w, stream=None) -> None:
    cb, pb = uq_packed_size(lay)
    _check("uq_dequant", _lib.uq_dequant(ctypes.byref(lay), _ptr(codes, "codes", cb, _U8),
                                         _ptr(params, "params", pb, _F16 + ("int32",)),
                                         _ptr(w, "w", lay.n * lay.k * 4, _F32), _stream(stream)))


def uq_rope_table(theta: float, head_dim: int, max_pos: int) -> tuple[np.ndarray, np.ndarray]:
    """Host rotary table: (cos, sin), each fp32 [max_pos, head_dim // 2]."""
    cos = np.empty((max_pos, head_dim // 2), dtype=np.float32)
    sin = np.empty_like(cos)
    _check("uq_rope_table", _lib.uq_rope_table(float(theta), int(head_dim), int(max_pos),
                                               cos.ctypes.data, sin.ctypes.data))
    return cos, sin


def uq_rmsnorm_rope(x, y, gamma, pos, cos, sin, tokens: int, heads: int, head_dim: int, max_pos: int,
                    eps: float, stream=None) -> None:
    """Fused RMSNorm + RoPE on device buffers (x, y fp16 [tokens, heads, head_dim]; y may be x)."""
    vec = max(int(tokens), 0) * max(int(heads), 0) * max(int(head_dim), 0) * 2
    tab = max(int(max_pos), 0) * max(int(head_dim), 0) // 2 * 4
    _check("uq_rmsnorm_rope", _lib.uq_rmsnorm_rope(
        _ptr(x, "x", vec, _F16), _ptr(y, "y", vec, _F16), _ptr(gamma, "gamma", 4 * max(int(head_dim), 0), _F32),
        _ptr(pos, "pos", 4 * max(int(tokens), 0), ("int32",)), _ptr(cos, "cos", tab, _F32),
        _ptr(sin, "sin", tab, _F32), int(tokens), int(heads), int(head_dim), int(max_pos), float(eps),
        _stream(stream)))


def uq_probe_read(src, nbytes: int, workgroups: int, loads_in_flight: int, sink, stream=None) -> None:
    """Measurement hook: read nbytes of src once with the GEMV's load pattern."""
    _check("uq_probe_read", _lib.uq_probe_read(_ptr(src, "src", int(nbytes)), int(nbytes), int(workgroups),
                                               int(loads_in_flight), _ptr(sink, "sink", 16 * int(workgroups)),
                                               _stream(stream)))


def uq_nf4_codebook() -> np.ndarray:
    out = np.empty(16, dtype=np.float32)
    _check("uq_nf4_codebook", _lib.uq_nf4_codebook(out.ctypes.data))
    return out


def uq_status_str(code: int) -> str:
    return _lib.uq_status_str(int(code)).decode()


def raw_call(name: str, *args) -> int:
    """Call an entry point with raw ctypes arguments and return its status (tests of error paths)."""
    return getattr(_lib, name)(*args)
