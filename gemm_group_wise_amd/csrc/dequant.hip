// Whole-matrix dequantization to fp32 (the matching dequantizer of
// "Ultra LLM Engine", Core Components > Quantization).  One thread per
// 16-byte code chunk; INT-N: w' = fma(q, s, z) (a single rounding of q*s + z);
// NF4: w' = C[q] * a.
#include "device_common.hpp"

namespace uq {
namespace {

template <int S>
__device__ __forceinline__ uint32_t code_at(const uint4& v, int i) {
  constexpr int bits = Fmt<S>::bits;
  constexpr int per_dword = 32 / bits;
  const uint32_t d = i / per_dword == 0 ? v.x : i / per_dword == 1 ? v.y : i / per_dword == 2 ? v.z : v.w;
  return (d >> (bits * (i % per_dword))) & ((1u << bits) - 1u);
}

template <int S, int G>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ params,
                                                      float* __restrict__ w, int64_t n_chunks,
                                                      int64_t chunks_per_row, int ng) {
  constexpr int CW = Fmt<S>::CW;
  const int64_t ch = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (ch >= n_chunks) return;
  const int64_t row = ch / chunks_per_row, cc = ch - row * chunks_per_row;
  const uint4 v = *reinterpret_cast<const uint4*>(codes + ch * 16);
  float out[CW];
#pragma unroll
  for (int i = 0; i < CW; ++i) {
    const uint32_t q = code_at<S>(v, i);
    const int64_t g = row * ng + (cc * CW + i) / G;
    if constexpr (S == UQ_NF4) {
      const float a = h2f(*reinterpret_cast<const uint16_t*>(params + g * 2));
      out[i] = nf4_value(int(q)) * a;
    } else {
      const uint32_t p = *reinterpret_cast<const uint32_t*>(params + g * 4);
      out[i] = __builtin_fmaf(float(q), h2f(uint16_t(p & 0xFFFFu)), h2f(uint16_t(p >> 16)));
    }
  }
  float4* dst = reinterpret_cast<float4*>(w + ch * CW);
#pragma unroll
  for (int i = 0; i < CW / 4; ++i) dst[i] = make_float4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
}

template <int S, int G>
hipError_t launch(const uq_layout* L, const void* codes, const void* params, float* w, hipStream_t stream) {
  constexpr int CW = Fmt<S>::CW;
  int64_t chunks_per_row = L->k / CW;
  int64_t n_chunks = L->n * chunks_per_row;
  int ng = int(L->k / G);
  const uint8_t* c8 = static_cast<const uint8_t*>(codes);
  const uint8_t* p8 = static_cast<const uint8_t*>(params);
  void* args[] = {&c8, &p8, &w, &n_chunks, &chunks_per_row, &ng};
  const int64_t blocks = (n_chunks + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid{unsigned(blocks)}, block{256};
  return hipLaunchKernel(reinterpret_cast<const void*>(&dequant_kernel<S, G>), grid, block, args, 0, stream);
}

}  // namespace

hipError_t launch_dequant(const uq_layout* L, const void* codes, const void* params, float* w,
                          hipStream_t stream) {
  switch (L->scheme * 1000 + L->group) {
    case UQ_INT2 * 1000 + 16: return launch<UQ_INT2, 16>(L, codes, params, w, stream);
    case UQ_INT2 * 1000 + 32: return launch<UQ_INT2, 32>(L, codes, params, w, stream);
    case UQ_INT2 * 1000 + 64: return launch<UQ_INT2, 64>(L, codes, params, w, stream);
    case UQ_INT2 * 1000 + 128: return launch<UQ_INT2, 128>(L, codes, params, w, stream);
    case UQ_INT4 * 1000 + 32: return launch<UQ_INT4, 32>(L, codes, params, w, stream);
    case UQ_INT4 * 1000 + 64: return launch<UQ_INT4, 64>(L, codes, params, w, stream);
    case UQ_INT4 * 1000 + 128: return launch<UQ_INT4, 128>(L, codes, params, w, stream);
    case UQ_INT8 * 1000 + 32: return launch<UQ_INT8, 32>(L, codes, params, w, stream);
    case UQ_INT8 * 1000 + 64: return launch<UQ_INT8, 64>(L, codes, params, w, stream);
    case UQ_INT8 * 1000 + 128: return launch<UQ_INT8, 128>(L, codes, params, w, stream);
    case UQ_NF4 * 1000 + 64: return launch<UQ_NF4, 64>(L, codes, params, w, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace uq
