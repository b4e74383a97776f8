// Internal definitions shared by the host packer, the C ABI and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "uq.h"

namespace uq {

// NormalFloat4 codebook (QLoRA construction: standard-normal quantiles at
// 8 equally spaced probabilities from p* = 0.9677083 down to 0.5 for the
// positive side, 7 for the negative side, plus 0, scaled to [-1, 1]); fp32
// bit patterns, index 0 -> 15.  "Ultra LLM Engine", Core Components >
// Quantization, nf4 row.
static constexpr uint32_t kNf4Bits[16] = {
    0xbf800000u, 0xbf3239b3u, 0xbf066b30u, 0xbeca32a0u,
    0xbe91a24cu, 0xbe3d353fu, 0xbdba786bu, 0x00000000u,
    0x3da2fb03u, 0x3e24cae1u, 0x3e7c04dcu, 0x3ead0338u,
    0x3ee1a4b7u, 0x3f1007aau, 0x3f3913b1u, 0x3f800000u};

// Code width in bits per scheme; 0 for an unknown scheme.
constexpr int scheme_bits(int scheme) {
  return scheme == UQ_INT2 ? 2
       : scheme == UQ_INT4 ? 4
       : scheme == UQ_INT8 ? 8
       : scheme == UQ_NF4  ? 4
                           : 0;
}

constexpr bool group_supported(int scheme, int g) {
  return scheme == UQ_INT2 ? (g == 16 || g == 32 || g == 64 || g == 128)
       : scheme == UQ_INT4 ? (g == 32 || g == 64 || g == 128)
       : scheme == UQ_INT8 ? (g == 32 || g == 64 || g == 128)
       : scheme == UQ_NF4  ? (g == 64)
                           : false;
}

// Bytes of one group's parameters: (s, z) fp16 pair, or one fp16 absmax.
constexpr int param_bytes_per_group(int scheme) { return scheme == UQ_NF4 ? 2 : 4; }

constexpr int64_t kMaxK = int64_t(1) << 24;
constexpr int64_t kMaxN = 0x7fffffff;

// Shape/format validation common to every entry point.
inline uq_status check_layout(const uq_layout* L) {
  if (!L) return UQ_ERR_NULL;
  const int bits = scheme_bits(L->scheme);
  if (!bits) return UQ_ERR_UNSUPPORTED;
  if (!group_supported(L->scheme, L->group)) return UQ_ERR_UNSUPPORTED;
  if (L->n < 1 || L->n > kMaxN) return UQ_ERR_SHAPE;
  if (L->k < 1 || L->k > kMaxK) return UQ_ERR_SHAPE;
  if (L->k % L->group) return UQ_ERR_SHAPE;
  if ((L->k * bits) % 128) return UQ_ERR_SHAPE;  // whole 16-byte code chunks
  return UQ_OK;
}

inline size_t code_row_bytes(const uq_layout* L) {
  return size_t(L->k) * size_t(scheme_bits(L->scheme)) / 8;
}
inline size_t param_row_bytes(const uq_layout* L) {
  return size_t(L->k / L->group) * size_t(param_bytes_per_group(L->scheme));
}

// Host packer (uq_pack.cpp).
uq_status pack_weights(const uq_layout* L, const float* w, uint8_t* codes,
                       uint16_t* params);

// Host re-layout of GGUF Q4_0 / Q8_0 blocks into the INT4 / INT8 G = 32 layout (uq_gguf.cpp).
uq_status import_gguf(int32_t type, const void* blocks, int64_t n, int64_t k, uq_layout* L,
                      uint8_t* codes, uint16_t* params);

// Host rotary table (rope_table.cpp).
uq_status rope_table(double theta, int32_t head_dim, int64_t max_pos, float* cos_out, float* sin_out);

// Head dimensions the fused RMSNorm + RoPE kernel serves.
constexpr bool rope_head_dim_supported(int32_t d) { return d == 64 || d == 128 || d == 256 || d == 512; }

}  // namespace uq
