// Argument checks of the device entry points of include/uq.h.  Host code
// only: every check here runs before the entry point makes its first HIP
// call, and on failure nothing is launched or written (the hard-fail stance
// of the lollms page, Vision item 3, and of the Ultra LLM Engine loader,
// Checkpoint Loading: refuse, never guess).
#include "uq_internal.h"

namespace uq {
namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

uq_status check_product(const uq_layout* L, const void* codes, const void* params, const void* x,
                        const void* y, int64_t m, int64_t mmax) {
  const uq_status st = check_layout(L);
  if (st != UQ_OK) return st;
  if (!codes || !params || !x || !y) return UQ_ERR_NULL;
  if (m < 1 || m > mmax) return UQ_ERR_SHAPE;
  if (!aligned(codes, 16) || !aligned(params, 16) || !aligned(x, 16) || !aligned(y, 16)) return UQ_ERR_ALIGN;
  return UQ_OK;
}

uq_status check_gemm_workspace(const uq_layout* L, int64_t m, const void* workspace, size_t bytes) {
  const size_t need = gemm_workspace(L, m).total;
  if (!workspace) return UQ_ERR_NULL;
  if (!aligned(workspace, 256)) return UQ_ERR_ALIGN;
  if (bytes < need) return UQ_ERR_WORKSPACE;
  return UQ_OK;
}

uq_status check_dequant(const uq_layout* L, const void* codes, const void* params, const void* w) {
  const uq_status st = check_layout(L);
  if (st != UQ_OK) return st;
  if (!codes || !params || !w) return UQ_ERR_NULL;
  if (!aligned(codes, 16) || !aligned(params, 16) || !aligned(w, 16)) return UQ_ERR_ALIGN;
  return UQ_OK;
}

uq_status check_quantize_activations(int32_t group, const void* x, const void* q, const void* sx, int64_t m,
                                     int64_t k) {
  if (!x || !q || !sx) return UQ_ERR_NULL;
  if (group != 16 && group != 32 && group != 64 && group != 128) return UQ_ERR_UNSUPPORTED;
  if (m < 1 || m > UQ_GEMM_MAX_M || k < 16 || k > kMaxK || k % group || k % 16) return UQ_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(sx, 4)) return UQ_ERR_ALIGN;
  return UQ_OK;
}

uq_status check_rmsnorm_rope(const void* x, const void* y, const void* gamma, const void* pos, const void* cos,
                             const void* sin, int64_t tokens, int32_t heads, int32_t head_dim, int64_t max_pos,
                             float eps) {
  if (!x || !y || !gamma || !pos || !cos || !sin) return UQ_ERR_NULL;
  if (!rope_head_dim_supported(head_dim)) return UQ_ERR_UNSUPPORTED;
  if (tokens < 0 || heads < 1 || max_pos < 1 || max_pos > (int64_t(1) << 24)) return UQ_ERR_SHAPE;
  if (tokens > (int64_t(1) << 40) / (int64_t(heads) * head_dim)) return UQ_ERR_SHAPE;
  if (!(eps >= 0.0f) || !(eps <= 3.4e38f)) return UQ_ERR_RANGE;  // also rejects NaN
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(gamma, 16) || !aligned(cos, 16) || !aligned(sin, 16) ||
      !aligned(pos, 4))
    return UQ_ERR_ALIGN;
  return UQ_OK;
}

uq_status check_probe_read(const void* src, size_t bytes, int32_t workgroups, int32_t loads_in_flight,
                           const void* sink) {
  if ((!src && bytes) || !sink) return UQ_ERR_NULL;
  if (bytes % 1024 || workgroups < 1 || workgroups > (1 << 20)) return UQ_ERR_SHAPE;
  if (loads_in_flight != 4 && loads_in_flight != 8 && loads_in_flight != 16 && loads_in_flight != 32)
    return UQ_ERR_UNSUPPORTED;
  if (!aligned(src, 16) || !aligned(sink, 4)) return UQ_ERR_ALIGN;
  return UQ_OK;
}

}  // namespace uq
