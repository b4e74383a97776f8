"""gemm_group_wise_amd -- fused group-wise dequant + GEMV/GEMM (and the fused
RMSNorm + RoPE step) for MI355X (gfx950).

The compute lives in ``libuq.so`` (HIP kernels behind the C ABI of
``include/uq.h``); this package is its thin Python binding.  Importing it
without a built library raises ImportError.
"""
from ._binding import (  # noqa: F401
    BITS, EXPORTS, GEMM_MAX_M, GEMV_MAX_M, LIB_PATH, SCHEMES, STATUS, Layout, UQError,
    GGUF_TYPES, gemm_workspace, layout, raw_call, uq_dequant, uq_gemm, uq_gemm_noalloc, uq_gemm_workspace_size, GEMM_NOALLOC_MAX_BYTES, uq_gemv, uq_gemv_a8, uq_import_gguf, uq_nf4_codebook,
    uq_pack_weights, uq_probe_read,
    uq_packed_size, uq_quantize_activations, uq_rmsnorm_rope, uq_rope_table, uq_status_str,
)
