// Dispatch of the fused dequant + GEMV kernel by scheme; the kernel itself is in
// gemv_impl.hpp and each scheme is instantiated in its own file (gemv_*.hip).
#include <hip/hip_runtime.h>

#include "uq_internal.h"

namespace uq {

#define UQ_GEMV_DECL(name)                                                                        \
  hipError_t launch_gemv_##name(const uq_layout* L, const void* codes, const void* params,       \
                                const uint16_t* x, float* y, int m, hipStream_t stream);
UQ_GEMV_DECL(int2)
UQ_GEMV_DECL(int4)
UQ_GEMV_DECL(int8)
UQ_GEMV_DECL(nf4)
#undef UQ_GEMV_DECL

hipError_t launch_gemv(const uq_layout* L, const void* codes, const void* params, const uint16_t* x,
                       float* y, int m, hipStream_t stream) {
  switch (L->scheme) {
    case UQ_INT2: return launch_gemv_int2(L, codes, params, x, y, m, stream);
    case UQ_INT4: return launch_gemv_int4(L, codes, params, x, y, m, stream);
    case UQ_INT8: return launch_gemv_int8(L, codes, params, x, y, m, stream);
    case UQ_NF4: return launch_gemv_nf4(L, codes, params, x, y, m, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace uq
