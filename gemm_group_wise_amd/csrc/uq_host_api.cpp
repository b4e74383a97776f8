// Host-only entry points of include/uq.h: sizes, the packer, the GGUF
// re-layout, the rotary table, the codebook and status names.  Plain C++ (no
// HIP): none of these touches a device.
#include <cstring>

#include "uq_internal.h"

extern "C" {

uq_status uq_packed_size(const uq_layout* layout, size_t* code_bytes, size_t* param_bytes) {
  const uq_status st = uq::check_layout(layout);
  if (st != UQ_OK) return st;
  if (!code_bytes || !param_bytes) return UQ_ERR_NULL;
  *code_bytes = uq::code_row_bytes(layout) * size_t(layout->n);
  *param_bytes = uq::param_row_bytes(layout) * size_t(layout->n);
  return UQ_OK;
}

uq_status uq_gemm_workspace_size(const uq_layout* layout, int64_t m, size_t* bytes) {
  const uq_status st = uq::check_layout(layout);
  if (st != UQ_OK) return st;
  if (!bytes) return UQ_ERR_NULL;
  if (m < 1 || m > UQ_GEMM_MAX_M) return UQ_ERR_SHAPE;
  *bytes = uq::gemm_workspace(layout, m).total;
  return UQ_OK;
}

uq_status uq_pack_weights(const uq_layout* layout, const float* w, uint8_t* codes, uint16_t* params) {
  return uq::pack_weights(layout, w, codes, params);
}

uq_status uq_import_gguf(int32_t gguf_type, const void* blocks, int64_t n, int64_t k, uq_layout* layout,
                         uint8_t* codes, uint16_t* params) {
  return uq::import_gguf(gguf_type, blocks, n, k, layout, codes, params);
}

uq_status uq_rope_table(double theta, int32_t head_dim, int64_t max_pos, float* cos, float* sin) {
  return uq::rope_table(theta, head_dim, max_pos, cos, sin);
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
    case UQ_ERR_WORKSPACE: return "UQ_ERR_WORKSPACE";
  }
  return "UQ_ERR_UNKNOWN";
}

}  // extern "C"
