// Rotary table for the fused RMSNorm + RoPE step ("Ultra LLM Engine", Core
// Components > Fused Kernels, third bullet).  Pair i of a head_dim-long vector
// turns by p * theta^(-2i/head_dim) at position p; the table holds the fp32
// cosine and sine of that angle, formed in fp64 and rounded once.
#include <cmath>

#include "uq_internal.h"

namespace uq {

uq_status rope_table(double theta, int32_t head_dim, int64_t max_pos, float* cos_out, float* sin_out) {
  if (!cos_out || !sin_out) return UQ_ERR_NULL;
  if (head_dim < 2 || head_dim % 2 || max_pos < 1 || max_pos > (int64_t(1) << 24) || !(theta > 0) ||
      !std::isfinite(theta))
    return UQ_ERR_SHAPE;
  const int32_t h = head_dim / 2;
  for (int32_t i = 0; i < h; ++i) {
    const double inv_freq = std::pow(theta, -2.0 * double(i) / double(head_dim));
    for (int64_t p = 0; p < max_pos; ++p) {
      const double a = double(p) * inv_freq;
      cos_out[p * h + i] = float(std::cos(a));
      sin_out[p * h + i] = float(std::sin(a));
    }
  }
  return UQ_OK;
}

}  // namespace uq
