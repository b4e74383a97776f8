// INT4 instantiations of the fused dequant + GEMV kernel (gemv_impl.hpp).
#include "gemv_impl.hpp"
#include "gemv_mfma.hpp"

namespace uq {

hipError_t launch_gemv_int4(const uq_layout* L, const void* codes, const void* params,
                         const uint16_t* x, float* y, int m, hipStream_t stream) {
  switch (L->group) {
    case 32: return launch_gemv_sel<UQ_INT4, 32>(L, codes, params, x, y, m, stream);
    case 64: return launch_gemv_sel<UQ_INT4, 64>(L, codes, params, x, y, m, stream);
    case 128: return launch_gemv_sel<UQ_INT4, 128>(L, codes, params, x, y, m, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace uq
