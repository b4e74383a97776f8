// Fused RMSNorm followed by RoPE ("Ultra LLM Engine", Core Components > Fused
// Kernels, third bullet; the Architecture diagram's "RMSNorm + RoPE" step).
//
//   u = x / sqrt(mean(x^2) + eps) * gamma                 over one vector of D
//   y[i] = u[i] c - u[i+h] s,  y[i+h] = u[i+h] c + u[i] s,  h = D/2,
//   c, s = cos/sin table row of the vector's token position.
//
// HBM-bound elementwise work: each vector is read once (fp16) and written once
// (fp16); gamma and the table rows are shared by all heads of a token and stay
// in cache.  A vector of D values is spread over L = D/8 lanes, 8 values (one
// 16-byte load) per lane, so one wave holds 64/L vectors; the sum of squares
// is reduced across the L lanes with lane swaps, and the rotation partner of
// lane j's values (index + D/2) sits in lane j + L/2, one more swap away.
// Everything is computed in fp32 and rounded to fp16 once.
#include <hip/hip_runtime.h>

#include "uq_internal.h"

namespace uq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <int D>
// x and y may be the same buffer (in place): neither is declared __restrict__.
// Each value is read once, before the lane that read it writes it.
__global__ __launch_bounds__(256) void rmsnorm_rope_kernel(const uint16_t* x, uint16_t* y,
                                                           const float* __restrict__ gamma,
                                                           const int32_t* __restrict__ pos,
                                                           const float* __restrict__ cos_tab,
                                                           const float* __restrict__ sin_tab, int64_t vectors,
                                                           int32_t heads, int64_t max_pos, float eps) {
  constexpr int L = D / 8;       // lanes per vector
  constexpr int VPW = 64 / L;    // vectors per wave
  constexpr int H = D / 2;
  const int lane = threadIdx.x & 63;
  const int j = lane % L;        // this lane's 8 values: [8j, 8j + 8)
  const int jr = j % (L / 2);    // their pair index block: [8jr, 8jr + 8) of the h pairs
  const float sign = j < L / 2 ? -1.0f : 1.0f;

  // gamma for this lane's 8 values
  const float4 g0 = reinterpret_cast<const float4*>(gamma)[2 * j];
  const float4 g1 = reinterpret_cast<const float4*>(gamma)[2 * j + 1];
  const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};

  const int64_t wave = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = (int64_t(gridDim.x) * blockDim.x) >> 6;
  for (int64_t v0 = wave * VPW; v0 < vectors; v0 += nwaves * VPW) {
    const int64_t v = v0 + lane / L;
    const bool live = v < vectors;
    const int64_t vc = live ? v : vectors - 1;   // past the end: recompute the last vector, store nothing
    const int64_t t = vc / heads;
    const int32_t p = pos[t];
    const bool in_range = p >= 0 && int64_t(p) < max_pos;
    const int64_t pc = in_range ? p : 0;          // never read outside the table

    const uint4 raw = reinterpret_cast<const uint4*>(x + vc * D)[j];
    const f16x8 xh = __builtin_bit_cast(f16x8, raw);
    float xv[8];
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      xv[e] = float(xh[e]);
      ss = __builtin_fmaf(xv[e], xv[e], ss);
    }
#pragma unroll
    for (int off = L / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
    const float r = 1.0f / __builtin_sqrtf(ss * (1.0f / float(D)) + eps);

    const float4* crow = reinterpret_cast<const float4*>(cos_tab + pc * H) + 2 * jr;
    const float4* srow = reinterpret_cast<const float4*>(sin_tab + pc * H) + 2 * jr;
    const float4 c0 = crow[0], c1 = crow[1], s0 = srow[0], s1 = srow[1];
    const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};

    f16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float u = xv[e] * r * g[e];
      const float partner = __shfl_xor(u, L / 2, 64);   // value e of lane j +- L/2: index +- D/2
      const float yv = __builtin_fmaf(sign * partner, s[e], u * c[e]);
      out[e] = _Float16(in_range ? yv : __builtin_nanf(""));
    }
    if (live) reinterpret_cast<uint4*>(y + vc * D)[j] = __builtin_bit_cast(uint4, out);
  }
}

template <int D>
hipError_t launch_d(const uint16_t* x, uint16_t* y, const float* gamma, const int32_t* pos, const float* c,
                    const float* s, int64_t tokens, int32_t heads, int64_t max_pos, float eps, hipStream_t stream) {
  int64_t vectors = tokens * int64_t(heads);
  constexpr int VPB = 4 * (64 / (D / 8));  // vectors per 256-thread block pass
  int64_t blocks = (vectors + VPB - 1) / VPB;
  if (blocks > 65536) blocks = 65536;      // the loop strides over the rest
  void* args[] = {(void*)&x, &y, (void*)&gamma, (void*)&pos, (void*)&c, (void*)&s, &vectors, &heads, &max_pos, &eps};
  return hipLaunchKernel(reinterpret_cast<const void*>(&rmsnorm_rope_kernel<D>), dim3(unsigned(blocks)), dim3(256),
                         args, 0, stream);
}

}  // namespace

hipError_t launch_rmsnorm_rope(const uint16_t* x, uint16_t* y, const float* gamma, const int32_t* pos,
                               const float* cos_tab, const float* sin_tab, int64_t tokens, int32_t heads,
                               int32_t head_dim, int64_t max_pos, float eps, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_d<64>(x, y, gamma, pos, cos_tab, sin_tab, tokens, heads, max_pos, eps, stream);
    case 128: return launch_d<128>(x, y, gamma, pos, cos_tab, sin_tab, tokens, heads, max_pos, eps, stream);
    case 256: return launch_d<256>(x, y, gamma, pos, cos_tab, sin_tab, tokens, heads, max_pos, eps, stream);
    case 512: return launch_d<512>(x, y, gamma, pos, cos_tab, sin_tab, tokens, heads, max_pos, eps, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace uq
