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

// fp16 with biased exponent E and a zero mantissa is 2^(E-15); OR-ing an
// integer c < 1024 into the 10-bit mantissa gives 2^(E-15) * (1 + c/1024).
// A code q left in place at mantissa bit b (c = q << b) therefore reads as
// exactly B + q when the base is B = 2^(10-b): 1024 (0x6400) for bit 0, 256
// (0x5C00) for bit 2, 64 (0x5400) for bit 4, 16 (0x4C00) for bit 6.  The
// unpackers below mask codes where they sit, two codes per fp16 pair, with one
// AND-OR per pair and the base that matches the bit position, so every pair
// is (B + q_a, B + q_b) exactly and the activations are used as they come;
// the per-group correction removes B * sum x.
constexpr uint32_t kMagic2 = 0x64006400u;  // base 1024, code at bit 0 of each half
constexpr uint32_t kBase256 = 0x5C005C00u, kBase64 = 0x54005400u, kBase16 = 0x4C004C00u;

// Position of dword-local code i among the pairs: pair j, half h; base of pair j.
template <int S> struct Slot;
template <> struct Slot<UQ_INT4> {
  // pairs: 0 = (c0, c4), 1 = (c2, c6) base 1024; 2 = (c1, c5), 3 = (c3, c7) base 64
  static __host__ __device__ constexpr int pair(int i) { return (i & 1) ? 2 + ((i & 3) >> 1) : ((i & 3) >> 1); }
  static __host__ __device__ constexpr int half(int i) { return i >> 2; }
  static __host__ __device__ constexpr float base(int j) { return j < 2 ? 1024.0f : 64.0f; }
};
template <> struct Slot<UQ_INT2> {
  // pair j = (c_j, c_{j+8}) with base 1024 / 4^(j mod 4)
  static __host__ __device__ constexpr int pair(int i) { return i & 7; }
  static __host__ __device__ constexpr int half(int i) { return i >> 3; }
  static __host__ __device__ constexpr float base(int j) {
    return (j & 3) == 0 ? 1024.0f : (j & 3) == 1 ? 256.0f : (j & 3) == 2 ? 64.0f : 16.0f;
  }
};
template <> struct Slot<UQ_INT8> {
  // pair j = (c_{2j}, c_{2j+1})
  static __host__ __device__ constexpr int pair(int i) { return i >> 1; }
  static __host__ __device__ constexpr int half(int i) { return i & 1; }
  static __host__ __device__ constexpr float base(int) { return 1024.0f; }
};
template <> struct Slot<UQ_NF4> {
  static __host__ __device__ constexpr int pair(int i) { return i >> 1; }
  static __host__ __device__ constexpr int half(int i) { return i & 1; }
  static __host__ __device__ constexpr float base(int) { return 0.0f; }  // codebook lookup, no base
};

// (a & mask) | orv in one v_and_or_b32.  gfx9 VOP3 encodings take no literal
// and at most one SGPR, so left to itself the compiler splits this into an
// AND and an OR with literals; here the mask rides in an SGPR and the magic
// constant in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t orv) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(orv));
  return r;
}

template <int S> __device__ __forceinline__ void unpack_pairs(uint32_t w, f16x2 (&p)[Fmt<S>::PPD]);

template <> __device__ __forceinline__ void unpack_pairs<UQ_INT4>(uint32_t w, f16x2 (&p)[4]) {
  const uint32_t w8 = w >> 8;
  p[0] = as_h2(and_or(w, 0x000F000Fu, kMagic2));
  p[1] = as_h2(and_or(w8, 0x000F000Fu, kMagic2));
  p[2] = as_h2(and_or(w, 0x00F000F0u, kBase64));
  p[3] = as_h2(and_or(w8, 0x00F000F0u, kBase64));
}

template <> __device__ __forceinline__ void unpack_pairs<UQ_INT2>(uint32_t w, f16x2 (&p)[8]) {
  const uint32_t w8 = w >> 8;
  constexpr uint32_t base[4] = {kMagic2, kBase256, kBase64, kBase16};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    p[j] = as_h2(and_or(w, 0x00030003u << (2 * j), base[j]));
    p[4 + j] = as_h2(and_or(w8, 0x00030003u << (2 * j), base[j]));
  }
}

template <> __device__ __forceinline__ void unpack_pairs<UQ_INT8>(uint32_t w, f16x2 (&p)[2]) {
  // v_perm_b32 selects bytes of {magic : w} (selector 0-3 = w, 4-7 = magic;
  // magic byte 5 is 0x64): (b0, 0x64, b1, 0x64) and (b2, 0x64, b3, 0x64)
  p[0] = as_h2(__builtin_amdgcn_perm(kMagic2, w, 0x05010500u));
  p[1] = as_h2(__builtin_amdgcn_perm(kMagic2, w, 0x05030502u));
}

// Activation pairing for the staged layout.  `d` holds WPD activations of one
// code dword in natural order as fp16 pairs d[j] = (x_{2j}, x_{2j+1}); the
// result is the PPD pairs the unpacker's output multiplies (a permutation
// only: the values are not scaled).  v_perm_b32 selector 0x05040100 takes the
// low halves of {S0 : S1}, 0x07060302 the high halves.
template <int S> __device__ __forceinline__ void pair_activations(const uint32_t (&d)[Fmt<S>::WPD / 2],
                                                                 f16x2 (&p)[Fmt<S>::PPD]);

template <> __device__ __forceinline__ void pair_activations<UQ_INT4>(const uint32_t (&d)[4], f16x2 (&p)[4]) {
  p[0] = as_h2(__builtin_amdgcn_perm(d[2], d[0], 0x05040100u));  // (x0, x4)
  p[1] = as_h2(__builtin_amdgcn_perm(d[3], d[1], 0x05040100u));  // (x2, x6)
  p[2] = as_h2(__builtin_amdgcn_perm(d[2], d[0], 0x07060302u));  // (x1, x5)
  p[3] = as_h2(__builtin_amdgcn_perm(d[3], d[1], 0x07060302u));  // (x3, x7)
}

template <> __device__ __forceinline__ void pair_activations<UQ_INT2>(const uint32_t (&d)[8], f16x2 (&p)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j)  // (x_j, x_{j+8})
    p[j] = as_h2(__builtin_amdgcn_perm(d[4 + j / 2], d[j / 2], (j & 1) ? 0x07060302u : 0x05040100u));
}

template <> __device__ __forceinline__ void pair_activations<UQ_INT8>(const uint32_t (&d)[2], f16x2 (&p)[2]) {
  p[0] = as_h2(d[0]);
  p[1] = as_h2(d[1]);
}

template <> __device__ __forceinline__ void pair_activations<UQ_NF4>(const uint32_t (&d)[4], f16x2 (&p)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) p[j] = as_h2(d[j]);
}

// DPP lane moves (gfx9 encodings).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum of each of four per-lane values over the 64 lanes of a wave, using the
// gfx950 lane-swap instructions as a transpose-reduction.  v_permlane32_swap
// exchanges the upper 32 lanes of its first operand with the lower 32 lanes of
// its second; v_permlane16_swap exchanges the odd 16-lane rows of the first
// with the even rows of the second.  Two levels of swap-and-add leave one
// register whose 16-lane rows hold partial sums of a, c, b, d (rows 0..3);
// DPP mirrors finish each row.  Result: lane 0 = sum(a), lane 16 = sum(c),
// lane 32 = sum(b), lane 48 = sum(d).
// The swaps are issued as inline asm with both registers in/out: the compiler
// builtins return the two swapped registers as a pair, and adding the pair's
// elements was compiled as the first element added to itself.  The compiler
// cannot see into the asm to pad its hazards, so the wait states around the
// cross-lane read and write are spelled out (generously).
__device__ __forceinline__ void permlane32_swap(float& x, float& y) {
  asm("s_nop 4\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 4" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ void permlane16_swap(float& x, float& y) {
  asm("s_nop 4\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 4" : "+v"(x), "+v"(y));
}

__device__ __forceinline__ float wave_sum4(float a, float b, float c, float d) {
  permlane32_swap(a, b);  // a = [a.lo32, b.lo32], b = [a.hi32, b.hi32]
  permlane32_swap(c, d);
  float s1 = a + b;       // lanes 0-31: a halves, lanes 32-63: b halves
  float s2 = c + d;
  permlane16_swap(s1, s2);
  float v = s1 + s2;      // 16-lane rows: a, c, b, d
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);  // row_half_mirror
  v += dpp_mov<0x140>(v);  // row_mirror
  return v;
}

// Loads of bytes a launch reads once (weight codes and group parameters):
// the non-temporal hint marks the lines for early eviction, so the stream
// does not push reused data (the activations) out of the caches.  Measured on
// the INT4 GEMV: about 5 % less time per launch.
template <typename T>
__device__ __forceinline__ T load_stream(const void* p) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  if constexpr (sizeof(T) == 16) {
    const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
    return T{v.x, v.y, v.z, v.w};
  } else if constexpr (sizeof(T) == 8) {
    const u32x2 v = __builtin_nontemporal_load(static_cast<const u32x2*>(p));
    return T{v.x, v.y};
  } else {
    return __builtin_nontemporal_load(static_cast<const T*>(p));
  }
}

// Device copy of the NF4 codebook (one per code object).
static __constant__ uint32_t kNf4Dev[16] = {
    kNf4Bits[0], kNf4Bits[1], kNf4Bits[2],  kNf4Bits[3],  kNf4Bits[4],  kNf4Bits[5],
    kNf4Bits[6], kNf4Bits[7], kNf4Bits[8],  kNf4Bits[9],  kNf4Bits[10], kNf4Bits[11],
    kNf4Bits[12], kNf4Bits[13], kNf4Bits[14], kNf4Bits[15]};

__device__ __forceinline__ float nf4_value(int i) { return __builtin_bit_cast(float, kNf4Dev[i]); }

__device__ __forceinline__ float h2f(uint16_t h) { return float(__builtin_bit_cast(_Float16, h)); }

}  // namespace uq
