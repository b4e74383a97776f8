// Device entry points of the C ABI (declared in include/uq.h): argument
// checks (uq_check.cpp, before any HIP call), kernel selection and launch on
// the caller's stream.  No entry point allocates device memory or
// synchronizes; uq_gemm works in the caller's workspace.
#include <hip/hip_runtime.h>

#include "uq_internal.h"

namespace uq {
hipError_t launch_gemv(const uq_layout* L, const void* codes, const void* params, const uint16_t* x,
                       float* y, int m, hipStream_t stream);
hipError_t launch_gemm(const uq_layout* L, const void* codes, const void* params, const uint16_t* x,
                       float* y, int m, void* workspace, hipStream_t stream);
hipError_t gemm_scratch(hipStream_t stream, void** out);
hipError_t launch_dequant(const uq_layout* L, const void* codes, const void* params, float* w,
                          hipStream_t stream);
hipError_t launch_gemv_a8(const uq_layout* L, const void* codes, const void* params, const uint16_t* x,
                          float* y, int m, hipStream_t stream);
hipError_t launch_quantize_a8(int32_t group, const uint16_t* x, int8_t* q, float* sx, int64_t m, int64_t k,
                              hipStream_t stream);
hipError_t launch_rmsnorm_rope(const uint16_t* x, uint16_t* y, const float* gamma, const int32_t* pos,
                               const float* cos_tab, const float* sin_tab, int64_t tokens, int32_t heads,
                               int32_t head_dim, int64_t max_pos, float eps, hipStream_t stream);

hipError_t launch_probe_read(const void* src, size_t bytes, int32_t workgroups, int32_t loads_in_flight,
                             uint32_t* sink, hipStream_t stream);

namespace {
uq_status launched(hipError_t e) { return e == hipSuccess ? UQ_OK : UQ_ERR_HIP; }
}  // namespace
}  // namespace uq

extern "C" {

uq_status uq_gemv(const uq_layout* layout, const void* codes, const void* params, const uint16_t* x, float* y,
                  int64_t m, void* stream) {
  const uq_status st = uq::check_product(layout, codes, params, x, y, m, UQ_GEMV_MAX_M);
  if (st != UQ_OK) return st;
  return uq::launched(uq::launch_gemv(layout, codes, params, x, y, int(m), static_cast<hipStream_t>(stream)));
}

uq_status uq_gemm(const uq_layout* layout, const void* codes, const void* params, const uint16_t* x, float* y,
                  int64_t m, void* workspace, size_t workspace_bytes, void* stream) {
  uq_status st = uq::check_product(layout, codes, params, x, y, m, UQ_GEMM_MAX_M);
  if (st != UQ_OK) return st;
  st = uq::check_gemm_workspace(layout, m, workspace, workspace_bytes);
  if (st != UQ_OK) return st;
  return uq::launched(
      uq::launch_gemm(layout, codes, params, x, y, int(m), workspace, static_cast<hipStream_t>(stream)));
}

uq_status uq_gemm_noalloc(const uq_layout* layout, const void* codes, const void* params, const uint16_t* x,
                          float* y, int64_t m, void* stream) {
  const uq_status st = uq::check_product(layout, codes, params, x, y, m, UQ_GEMM_MAX_M);
  if (st != UQ_OK) return st;
  if (uq::gemm_workspace(layout, m).total > uq::kGemmScratchBytes) return UQ_ERR_WORKSPACE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (uq::gemm_scratch(s, &ws) != hipSuccess) return UQ_ERR_HIP;
  return uq::launched(uq::launch_gemm(layout, codes, params, x, y, int(m), ws, s));
}

uq_status uq_dequant(const uq_layout* layout, const void* codes, const void* params, float* w, void* stream) {
  const uq_status st = uq::check_dequant(layout, codes, params, w);
  if (st != UQ_OK) return st;
  return uq::launched(uq::launch_dequant(layout, codes, params, w, static_cast<hipStream_t>(stream)));
}

uq_status uq_gemv_a8(const uq_layout* layout, const void* codes, const void* params, const uint16_t* x,
                     float* y, int64_t m, void* stream) {
  const uq_status st = uq::check_product(layout, codes, params, x, y, m, UQ_GEMV_MAX_M);
  if (st != UQ_OK) return st;
  if (layout->scheme == UQ_NF4) return UQ_ERR_UNSUPPORTED;
  return uq::launched(uq::launch_gemv_a8(layout, codes, params, x, y, int(m), static_cast<hipStream_t>(stream)));
}

uq_status uq_quantize_activations(int32_t group, const uint16_t* x, int8_t* q, float* sx, int64_t m, int64_t k,
                                  void* stream) {
  const uq_status st = uq::check_quantize_activations(group, x, q, sx, m, k);
  if (st != UQ_OK) return st;
  return uq::launched(uq::launch_quantize_a8(group, x, q, sx, m, k, static_cast<hipStream_t>(stream)));
}

uq_status uq_rmsnorm_rope(const uint16_t* x, uint16_t* y, const float* gamma, const int32_t* pos,
                          const float* cos, const float* sin, int64_t tokens, int32_t heads, int32_t head_dim,
                          int64_t max_pos, float eps, void* stream) {
  const uq_status st = uq::check_rmsnorm_rope(x, y, gamma, pos, cos, sin, tokens, heads, head_dim, max_pos, eps);
  if (st != UQ_OK) return st;
  if (tokens == 0) return UQ_OK;
  return uq::launched(uq::launch_rmsnorm_rope(x, y, gamma, pos, cos, sin, tokens, heads, head_dim, max_pos, eps,
                                              static_cast<hipStream_t>(stream)));
}

uq_status uq_probe_read(const void* src, size_t bytes, int32_t workgroups, int32_t loads_in_flight,
                        uint32_t* sink, void* stream) {
  const uq_status st = uq::check_probe_read(src, bytes, workgroups, loads_in_flight, sink);
  if (st != UQ_OK) return st;
  return uq::launched(
      uq::launch_probe_read(src, bytes, workgroups, loads_in_flight, sink, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
