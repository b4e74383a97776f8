// Device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "uq_internal.h"

namespace uq {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Packed-code geometry.  A "chunk" is the 16 bytes one lane loads with one
// 128-bit load; a dword of codes is the unit the unpackers work on.
template <int S> struct Fmt;
template <> struct Fmt<UQ_INT2> { static constexpr int bits = 2, CW = 64, WPD = 16, PPD = 8; };
template <> struct Fmt<UQ_INT4> { static constexpr int bits = 4, CW = 32, WPD = 8, PPD = 4; };
template <> struct Fmt<UQ_INT8> { static constexpr int bits = 8, CW = 16, WPD = 4, PPD = 2; };
template <> struct Fmt<UQ_NF4>  { static constexpr int bits = 4, CW = 32, WPD = 8, PPD = 4; };
// CW: codes per 16-byte chunk; WPD: codes per dword; PPD: fp16 pairs per dword.

__device__ __forceinline__ f16x2 as_h2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }
__device__ __forceinline__ uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// fp16 0x6400 is 1024.0 with a zero 10-bit mantissa: OR-ing an integer
// c < 1024 into the mantissa yields exactly 1024 + c.  The unpackers below
// turn a dword of codes into fp16 pairs (1024 + cls*q_a, 1024 + cls*q_b) with
// one AND-OR per pair, where cls is a power of two set by the bit position of
// the code; the activations are pre-divided by cls so the products carry the
// right weight, and the constant 1024 is removed with a per-group correction.
constexpr uint32_t kMagic2 = 0x64006400u;

// Position of dword-local code i among the pairs: pair j, half h, class cls.
template <int S> struct Slot;
template <> struct Slot<UQ_INT4> {
  // pairs: 0 = (c0, c4), 1 = (c2, c6), 2 = (c1, c5) x16, 3 = (c3, c7) x16
  static __host__ __device__ constexpr int pair(int i) { return (i & 1) ? 2 + ((i & 3) >> 1) : ((i & 3) >> 1); }
  static __host__ __device__ constexpr int half(int i) { return i >> 2; }
  static __host__ __device__ constexpr float inv_cls(int i) { return (i & 1) ? 0.0625f : 1.0f; }
};
template <> struct Slot<UQ_INT2> {
  // pair j = (c_j, c_{j+8}) scaled by 4^(j mod 4)
  static __host__ __device__ constexpr int pair(int i) { return i & 7; }
  static __host__ __device__ constexpr int half(int i) { return i >> 3; }
  static __host__ __device__ constexpr float inv_cls(int i) {
    return (i & 3) == 0 ? 1.0f : (i & 3) == 1 ? 0.25f : (i & 3) == 2 ? 0.0625f : 0.015625f;
  }
};
template <> struct Slot<UQ_INT8> {
  // pair j = (c_{2j}, c_{2j+1})
  static __host__ __device__ constexpr int pair(int i) { return i >> 1; }
  static __host__ __device__ constexpr int half(int i) { return i & 1; }
  static __host__ __device__ constexpr float inv_cls(int) { return 1.0f; }
};
template <> struct Slot<UQ_NF4> {
  static __host__ __device__ constexpr int pair(int i) { return i >> 1; }
  static __host__ __device__ constexpr int half(int i) { return i & 1; }
  static __host__ __device__ constexpr float inv_cls(int) { return 1.0f; }
};

template <int S> __device__ __forceinline__ void unpack_pairs(uint32_t w, f16x2 (&p)[Fmt<S>::PPD]);

template <> __device__ __forceinline__ void unpack_pairs<UQ_INT4>(uint32_t w, f16x2 (&p)[4]) {
  const uint32_t w8 = w >> 8;
  p[0] = as_h2((w & 0x000F000Fu) | kMagic2);
  p[1] = as_h2((w8 & 0x000F000Fu) | kMagic2);
  p[2] = as_h2((w & 0x00F000F0u) | kMagic2);
  p[3] = as_h2((w8 & 0x00F000F0u) | kMagic2);
}

template <> __device__ __forceinline__ void unpack_pairs<UQ_INT2>(uint32_t w, f16x2 (&p)[8]) {
  const uint32_t w8 = w >> 8;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    p[j] = as_h2((w & (0x00030003u << (2 * j))) | kMagic2);
    p[4 + j] = as_h2((w8 & (0x00030003u << (2 * j))) | kMagic2);
  }
}

template <> __device__ __forceinline__ void unpack_pairs<UQ_INT8>(uint32_t w, f16x2 (&p)[2]) {
  // v_perm_b32 picks bytes of {0x64646464 : w}: (b0, 0x64, b1, 0x64), (b2, 0x64, b3, 0x64)
  p[0] = as_h2(__builtin_amdgcn_perm(0x64646464u, w, 0x04010400u));
  p[1] = as_h2(__builtin_amdgcn_perm(0x64646464u, w, 0x04030402u));
}

// DPP lane moves (gfx9 encodings).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes of a wavefront; every lane receives the total.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);  // row_half_mirror
  v += dpp_mov<0x140>(v);  // row_mirror
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// Device copy of the NF4 codebook (one per code object).
static __constant__ uint32_t kNf4Dev[16] = {
    kNf4Bits[0], kNf4Bits[1], kNf4Bits[2],  kNf4Bits[3],  kNf4Bits[4],  kNf4Bits[5],
    kNf4Bits[6], kNf4Bits[7], kNf4Bits[8],  kNf4Bits[9],  kNf4Bits[10], kNf4Bits[11],
    kNf4Bits[12], kNf4Bits[13], kNf4Bits[14], kNf4Bits[15]};

__device__ __forceinline__ float nf4_value(int i) { return __builtin_bit_cast(float, kNf4Dev[i]); }

__device__ __forceinline__ float h2f(uint16_t h) { return float(__builtin_bit_cast(_Float16, h)); }

}  // namespace uq
