"""Reference oracle for group-wise weight quantization and dequant-GEMV/GEMM.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package.  The product path
(the HIP library and its Python binding) never imports it, and this package
imports nothing from the product path.
"""
from .uq_oracle import *  # noqa: F401,F403
from .uq_oracle import __all__  # noqa: F401
