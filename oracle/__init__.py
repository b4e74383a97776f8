"""Reference oracle for group-wise weight quantization, dequant-GEMV/GEMM, the
fused RMSNorm + RoPE step, the activation-quantized integer-dot GEMV and the
GGUF Q4_0 / Q8_0 block formats.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package.  The product path
(the HIP library and its Python binding) never imports it, and this package
imports nothing from the product path.
"""
from . import act_quant, gguf_blocks, norm_rope, uq_oracle
from .act_quant import *  # noqa: F401,F403
from .gguf_blocks import *  # noqa: F401,F403
from .norm_rope import *  # noqa: F401,F403
from .uq_oracle import *  # noqa: F401,F403

__all__ = (list(uq_oracle.__all__) + list(norm_rope.__all__) + list(act_quant.__all__)
           + list(gguf_blocks.__all__))
