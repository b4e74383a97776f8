// C ABI of libuq (declared in include/uq.h): argument validation, kernel
// selection and launch on the caller's stream.  Validation always precedes
// the first HIP call; no entry point synchronizes, and only uq_gemm allocates
// (its activation workspace, kept per device and stream).
#include <hip/hip_runtime.h>

#include <cstring>

#include "uq_internal.h"

namespace uq {
hipError_t launch_gemv(const uq_layout* L, const void* codes, const void* params, const uint16_t* x,
                       float* y, int m, hipStream_t stream);
hipError_t launch_gemm(const uq_layout* L, const void* codes, const void* params, const uint16_t* x,
                       float* y, int m, hipStream_t stream);
hipError_t launch_dequant(const uq_layout* L, const void* codes, const void* params, float* w,
                          hipStream_t stream);
hipError_t launch_gemv_a8(const uq_layout* L, const void* codes, const void* params, const uint16_t* x,
                          float* y, int m, hipStream_t stream);
hipError_t launch_quantize_a8(int32_t group, const uint16_t* x, int8_t* q, float* sx, int64_t m, int64_t k,
                              hipStream_t stream);
hipError_t launch_rmsnorm_rope(const uint16_t* x, uint16_t* y, const float* gamma, const int32_t* pos,
                               const float* cos_tab, const float* sin_tab, int64_t tokens, int32_t heads,
                               int32_t head_dim, int64_t max_pos, float eps, hipStream_t stream);

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

uq_status check_product(const uq_layout* L, const void* codes, const void* params, const void* x,
                        const void* y, int64_t m, int64_t mmax) {
  const uq_status st = check_layout(L);
  if (st != UQ_OK) return st;
  if (!codes || !params || !x || !y) return UQ_ERR_NULL;
  if (m < 1 || m > mmax) return UQ_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(params) || !aligned16(x) || !aligned16(y)) return UQ_ERR_ALIGN;
  return UQ_OK;
}

}  // namespace
}  // namespace uq

extern "C" {

uq_status uq_packed_size(const uq_layout* layout, size_t* code_bytes, size_t* param_bytes) {
  const uq_status st = uq::check_layout(layout);
  if (st != UQ_OK) return st;
  if (!code_bytes || !param_bytes) return UQ_ERR_NULL;
  *code_bytes = uq::code_row_bytes(layout) * size_t(layout->n);
  *param_bytes = uq::param_row_bytes(layout) * size_t(layout->n);
  return UQ_OK;
}

uq_status uq_pack_weights(const uq_layout* layout, const float* w, uint8_t* codes,
                          uint16_t* params) {
  return uq::pack_weights(layout, w, codes, params);
}

uq_status uq_import_gguf(int32_t gguf_type, const void* blocks, int64_t n, int64_t k, uq_layout* layout,
                         uint8_t* codes, uint16_t* params) {
  return uq::import_gguf(gguf_type, blocks, n, k, layout, codes, params);
}

uq_status uq_gemv(const uq_layout* layout, const void* codes, const void* params,
                  const uint16_t* x, float* y, int64_t m, void* stream) {
  const uq_status st = uq::check_product(layout, codes, params, x, y, m, UQ_GEMV_MAX_M);
  if (st != UQ_OK) return st;
  const hipError_t e =
      uq::launch_gemv(layout, codes, params, x, y, int(m), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? UQ_OK : UQ_ERR_HIP;
}

uq_status uq_gemm(const uq_layout* layout, const void* codes, const void* params,
                  const uint16_t* x, float* y, int64_t m, void* stream) {
  const uq_status st = uq::check_product(layout, codes, params, x, y, m, UQ_GEMM_MAX_M);
  if (st != UQ_OK) return st;
  const hipError_t e =
      uq::launch_gemm(layout, codes, params, x, y, int(m), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? UQ_OK : UQ_ERR_HIP;
}

uq_status uq_dequant(const uq_layout* layout, const void* codes, const void* params, float* w,
                     void* stream) {
  const uq_status st = uq::check_layout(layout);
  if (st != UQ_OK) return st;
  if (!codes || !params || !w) return UQ_ERR_NULL;
  if (!uq::aligned16(codes) || !uq::aligned16(params) || !uq::aligned16(w)) return UQ_ERR_ALIGN;
  const hipError_t e = uq::launch_dequant(layout, codes, params, w, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? UQ_OK : UQ_ERR_HIP;
}

uq_status uq_gemv_a8(const uq_layout* layout, const void* codes, const void* params,
                     const uint16_t* x, float* y, int64_t m, void* stream) {
  const uq_status st = uq::check_product(layout, codes, params, x, y, m, UQ_GEMV_MAX_M);
  if (st != UQ_OK) return st;
  if (layout->scheme == UQ_NF4) return UQ_ERR_UNSUPPORTED;
  const hipError_t e =
      uq::launch_gemv_a8(layout, codes, params, x, y, int(m), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? UQ_OK : UQ_ERR_HIP;
}

uq_status uq_quantize_activations(int32_t group, const uint16_t* x, int8_t* q, float* sx, int64_t m,
                                  int64_t k, void* stream) {
  if (!x || !q || !sx) return UQ_ERR_NULL;
  if (group != 16 && group != 32 && group != 64 && group != 128) return UQ_ERR_UNSUPPORTED;
  if (m < 1 || m > UQ_GEMM_MAX_M || k < 16 || k > uq::kMaxK || k % group || k % 16) return UQ_ERR_SHAPE;
  if (!uq::aligned16(x) || !uq::aligned16(q) || (reinterpret_cast<uintptr_t>(sx) & 3u)) return UQ_ERR_ALIGN;
  const hipError_t e = uq::launch_quantize_a8(group, x, q, sx, m, k, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? UQ_OK : UQ_ERR_HIP;
}

uq_status uq_rope_table(double theta, int32_t head_dim, int64_t max_pos, float* cos, float* sin) {
  return uq::rope_table(theta, head_dim, max_pos, cos, sin);
}

uq_status uq_rmsnorm_rope(const uint16_t* x, uint16_t* y, const float* gamma, const int32_t* pos,
                          const float* cos, const float* sin, int64_t tokens, int32_t heads,
                          int32_t head_dim, int64_t max_pos, float eps, void* stream) {
  if (!x || !y || !gamma || !pos || !cos || !sin) return UQ_ERR_NULL;
  if (!uq::rope_head_dim_supported(head_dim)) return UQ_ERR_UNSUPPORTED;
  if (tokens < 0 || heads < 1 || max_pos < 1 || max_pos > (int64_t(1) << 24)) return UQ_ERR_SHAPE;
  if (tokens > (int64_t(1) << 40) / (int64_t(heads) * head_dim)) return UQ_ERR_SHAPE;
  if (!(eps >= 0.0f) || !(eps <= 3.4e38f)) return UQ_ERR_RANGE;  // also rejects NaN
  if (!uq::aligned16(x) || !uq::aligned16(y) || !uq::aligned16(gamma) || !uq::aligned16(cos) ||
      !uq::aligned16(sin) || (reinterpret_cast<uintptr_t>(pos) & 3u))
    return UQ_ERR_ALIGN;
  if (tokens == 0) return UQ_OK;
  const hipError_t e = uq::launch_rmsnorm_rope(x, y, gamma, pos, cos, sin, tokens, heads, head_dim, max_pos, eps,
                                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? UQ_OK : UQ_ERR_HIP;
}

uq_status uq_nf4_codebook(float out[16]) {
  if (!out) return UQ_ERR_NULL;
  std::memcpy(out, uq::kNf4Bits, sizeof(uq::kNf4Bits));
  return UQ_OK;
}

const char* uq_status_str(uq_status status) {
  switch (status) {
    case UQ_OK: return "UQ_OK";
    case UQ_ERR_NULL: return "UQ_ERR_NULL";
    case UQ_ERR_SHAPE: return "UQ_ERR_SHAPE";
    case UQ_ERR_UNSUPPORTED: return "UQ_ERR_UNSUPPORTED";
    case UQ_ERR_ALIGN: return "UQ_ERR_ALIGN";
    case UQ_ERR_RANGE: return "UQ_ERR_RANGE";
    case UQ_ERR_HIP: return "UQ_ERR_HIP";
  }
  return "UQ_ERR_UNKNOWN";
}

}  // extern "C"
