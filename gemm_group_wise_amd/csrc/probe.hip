// Measurement hook: a plain streaming read, the ceiling the weight-streaming
// GEMV is compared against ("Ultra LLM Engine", Core Components > Fused
// Kernels: the decode GEMV is bound by reading the packed weights once).
//
// Every 16-byte word of [src, src + bytes) is read exactly once with the
// GEMV's access pattern: wave-wide 128-bit loads, each lane 16 bytes, so one
// load instruction reads 1 KB contiguously; the non-temporal hint the GEMV
// uses for its weights; a lane issues `UN` loads before it touches any of
// them.  Waves take contiguous runs of 1 KB blocks (`per_wave` blocks each,
// the last wave fewer), so the work per wave is as even as the byte count
// allows.  Each wave XORs what it read into one word of `sink` so the loads
// cannot be dropped.
#include <hip/hip_runtime.h>

#include "uq_internal.h"

namespace uq {
namespace {

template <int UN>
__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ src, int64_t blocks, int64_t per_wave,
                                                   uint32_t* __restrict__ sink) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int64_t wave = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t b0 = wave * per_wave;
  int64_t b1 = b0 + per_wave;
  b1 = b1 < blocks ? b1 : blocks;
  uint32_t acc = 0;
  for (int64_t b = b0; b < b1; b += UN) {
    u32x4 v[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int64_t bb = b + u < b1 ? b + u : b1 - 1;  // clamped: a valid block, read again
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + bb * 64 + lane));
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (b0 < b1) {
    // one word per wave: the XOR over its lanes
    for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
    if (lane == 0) sink[wave] = acc;
  }
}

}  // namespace

hipError_t launch_probe_read(const void* src, size_t bytes, int32_t workgroups, int32_t loads_in_flight,
                             uint32_t* sink, hipStream_t stream) {
  int64_t blocks = int64_t(bytes / 1024);
  const int64_t waves = int64_t(workgroups) * 4;
  int64_t per_wave = (blocks + waves - 1) / waves;
  const uint4* s = static_cast<const uint4*>(src);
  void* args[] = {(void*)&s, &blocks, &per_wave, &sink};
  const void* fn = loads_in_flight == 4    ? reinterpret_cast<const void*>(&read_kernel<4>)
                   : loads_in_flight == 8  ? reinterpret_cast<const void*>(&read_kernel<8>)
                   : loads_in_flight == 16 ? reinterpret_cast<const void*>(&read_kernel<16>)
                                           : reinterpret_cast<const void*>(&read_kernel<32>);
  return hipLaunchKernel(fn, dim3(unsigned(workgroups)), dim3(256), args, 0, stream);
}

}  // namespace uq
