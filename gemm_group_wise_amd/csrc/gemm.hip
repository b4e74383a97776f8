// Fused group-wise dequant + GEMM on the bf16 matrix cores, for batched
// decode and prefill ("Ultra LLM Engine", Core Components > Fused Kernels:
// dequantized-weight GEMM during batched decode).
//
// y[m][n] = sum_k bf16(x[m][k]) * bf16(w'[n][k]), fp32 accumulation, where
// w' = fma(q, s, z) (INT-N) or C[q] * a (NF4) is the exact fp32 dequant and
// both casts round to nearest even.
//
// Tiling: a workgroup of 4 waves computes a BM x 64 tile of y.  Per K step
// of 128 it dequantizes the 64 x 128 weight tile and converts the BM x 128
// activation tile to bf16 in LDS, then each wave runs v_mfma_f32_16x16x32_bf16
// on its sub-tile.  The blockIdx -> tile order keeps the M tiles of one
// weight tile on the same XCD, so their code reads share one L2.
#include "device_common.hpp"

namespace uq {
namespace {

constexpr int kBN = 64;
constexpr int kBK = 128;
constexpr int kPad = 8;  // bf16 elements of row padding in LDS
constexpr int kLd = kBK + kPad;

template <int S>
__device__ __forceinline__ uint32_t code_at(const uint32_t (&d)[8], int i) {
  constexpr int bits = Fmt<S>::bits;
  constexpr int per = 32 / bits;
  return (d[i / per] >> (bits * (i % per))) & ((1u << bits) - 1u);
}

// Dequantize 32 consecutive codes of one row (k0 .. k0+31) to bf16 in LDS.
template <int S, int G>
__device__ __forceinline__ void dequant32(const uint8_t* __restrict__ codes,
                                          const uint8_t* __restrict__ params, int row, int64_t k0,
                                          size_t rowb, int ng, __bf16* dst, const float* nf4) {
  constexpr int bits = Fmt<S>::bits;
  constexpr int nbytes = 32 * bits / 8;  // 8, 16 or 32
  uint32_t d[8];
  const uint8_t* src = codes + size_t(row) * rowb + size_t(k0) * bits / 8;
  if constexpr (nbytes == 8) {
    const uint2 v = *reinterpret_cast<const uint2*>(src);
    d[0] = v.x; d[1] = v.y;
  } else if constexpr (nbytes == 16) {
    const uint4 v = *reinterpret_cast<const uint4*>(src);
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
  } else {
    const uint4 v0 = *reinterpret_cast<const uint4*>(src);
    const uint4 v1 = *reinterpret_cast<const uint4*>(src + 16);
    d[0] = v0.x; d[1] = v0.y; d[2] = v0.z; d[3] = v0.w;
    d[4] = v1.x; d[5] = v1.y; d[6] = v1.z; d[7] = v1.w;
  }
  constexpr int NGP = G >= 32 ? 1 : 32 / G;  // groups spanned by the 32 codes
  float s[NGP], z[NGP];
  const int64_t g0 = int64_t(row) * ng + k0 / G;
#pragma unroll
  for (int j = 0; j < NGP; ++j) {
    if constexpr (S == UQ_NF4) {
      s[j] = h2f(*reinterpret_cast<const uint16_t*>(params + (g0 + j) * 2));
      z[j] = 0.0f;
    } else {
      const uint32_t p = *reinterpret_cast<const uint32_t*>(params + (g0 + j) * 4);
      s[j] = h2f(uint16_t(p & 0xFFFFu));
      z[j] = h2f(uint16_t(p >> 16));
    }
  }
  bf16x8 out[4];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t q = code_at<S>(d, i);
    const int j = i / (32 / NGP);
    float wv;
    if constexpr (S == UQ_NF4) wv = nf4[q] * s[j];
    else wv = __builtin_fmaf(float(q), s[j], z[j]);
    out[i / 8][i % 8] = __bf16(wv);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) *reinterpret_cast<bf16x8*>(dst + 8 * v) = out[v];
}

template <int S, int G, int BM>
__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t* __restrict__ codes,
                                                   const uint8_t* __restrict__ params,
                                                   const uint16_t* __restrict__ x,
                                                   float* __restrict__ y, int n, int k, int m,
                                                   int tiles_m, int tiles_n) {
  constexpr int WM = BM / 2;      // rows per wave (2 x 2 wave grid)
  constexpr int TM = WM / 16;     // 16-row MFMA tiles per wave
  constexpr int TN = 2;           // 16-col MFMA tiles per wave (32 cols)
  __shared__ __attribute__((aligned(16))) __bf16 As[BM * kLd];
  __shared__ __attribute__((aligned(16))) __bf16 Bs[kBN * kLd];
  __shared__ float nf4[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // Workgroups are dealt to the 8 XCDs round-robin (block b -> XCD b % 8).
  // Give XCD x the contiguous logical range [x * per_xcd, (x + 1) * per_xcd)
  // so the M tiles of one weight tile share an L2.
  const int total = tiles_m * tiles_n, per_xcd = (total + 7) / 8;
  const int logical = int(blockIdx.x % 8) * per_xcd + int(blockIdx.x / 8);
  if (logical >= total) return;
  const int tile_n = logical / tiles_m, tile_m = logical - tile_n * tiles_m;
  const int bm = tile_m * BM, bn = tile_n * kBN;
  const size_t rowb = size_t(k) * Fmt<S>::bits / 8;
  const int ng = k / G;
  if constexpr (S == UQ_NF4) {
    if (tid < 16) nf4[tid] = nf4_value(tid);
    __syncthreads();
  }

  f32x4 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < k; k0 += kBK) {
    // weight tile: 64 rows x 128 codes; thread -> (row, 32-code piece)
    {
      const int r = tid >> 2, pc = (tid & 3) * 32;
      const int row = bn + r < n ? bn + r : n - 1;
      if (k0 + pc < k) {
        dequant32<S, G>(codes, params, row, k0 + pc, rowb, ng, Bs + r * kLd + pc, nf4);
      } else {  // K tail (k is a multiple of 32): zero pieces past the end
#pragma unroll
        for (int v = 0; v < 4; ++v) *reinterpret_cast<uint4*>(Bs + r * kLd + pc + 8 * v) = make_uint4(0, 0, 0, 0);
      }
    }
    // activation tile: BM rows x 128, fp16 -> bf16
#pragma unroll
    for (int it = tid; it < BM * 4; it += 256) {
      const int r = it >> 2, pc = (it & 3) * 32;
      __bf16* dst = As + r * kLd + pc;
      if (bm + r < m && k0 + pc < k) {
        const uint4* src = reinterpret_cast<const uint4*>(x + size_t(bm + r) * size_t(k) + k0 + pc);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint4 raw = src[v];
          const uint16_t* h = reinterpret_cast<const uint16_t*>(&raw);
          bf16x8 o;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = __bf16(h2f(h[e]));
          *reinterpret_cast<bf16x8*>(dst + 8 * v) = o;
        }
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) *reinterpret_cast<uint4*>(dst + 8 * v) = make_uint4(0, 0, 0, 0);
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 32) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int a = 0; a < TM; ++a)
        af[a] = *reinterpret_cast<const bf16x8*>(As + (wm * WM + a * 16 + (lane & 15)) * kLd + kk + 8 * (lane >> 4));
#pragma unroll
      for (int b = 0; b < TN; ++b)
        bfr[b] = *reinterpret_cast<const bf16x8*>(Bs + (wn * 32 + b * 16 + (lane & 15)) * kLd + kk + 8 * (lane >> 4));
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
    }
    __syncthreads();
  }

  // D layout of a 16x16 tile: lane l holds rows 4*(l/16) + v, column l % 16.
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      const int col = bn + wn * 32 + b * 16 + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = bm + wm * WM + a * 16 + 4 * (lane >> 4) + v;
        if (row < m && col < n) y[size_t(row) * size_t(n) + col] = acc[a][b][v];
      }
    }
}

template <int S, int G, int BM>
hipError_t launch(const uq_layout* L, const void* codes, const void* params, const uint16_t* x,
                  float* y, int m, hipStream_t stream) {
  int n = int(L->n), k = int(L->k);
  int tiles_m = (m + BM - 1) / BM, tiles_n = (n + kBN - 1) / kBN;
  const uint8_t* c8 = static_cast<const uint8_t*>(codes);
  const uint8_t* p8 = static_cast<const uint8_t*>(params);
  void* args[] = {&c8, &p8, (void*)&x, &y, &n, &k, &m, &tiles_m, &tiles_n};
  const dim3 grid(unsigned(((tiles_m * tiles_n + 7) / 8) * 8)), block(256);
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_kernel<S, G, BM>), grid, block, args, 0, stream);
}

template <int S, int G>
hipError_t launch_bm(const uq_layout* L, const void* codes, const void* params, const uint16_t* x,
                     float* y, int m, hipStream_t stream) {
  if (m <= 32) return launch<S, G, 32>(L, codes, params, x, y, m, stream);
  return launch<S, G, 64>(L, codes, params, x, y, m, stream);
}

}  // namespace

hipError_t launch_gemm(const uq_layout* L, const void* codes, const void* params, const uint16_t* x,
                       float* y, int m, hipStream_t stream) {
  switch (L->scheme * 1000 + L->group) {
    case UQ_INT2 * 1000 + 16: return launch_bm<UQ_INT2, 16>(L, codes, params, x, y, m, stream);
    case UQ_INT2 * 1000 + 32: return launch_bm<UQ_INT2, 32>(L, codes, params, x, y, m, stream);
    case UQ_INT2 * 1000 + 64: return launch_bm<UQ_INT2, 64>(L, codes, params, x, y, m, stream);
    case UQ_INT2 * 1000 + 128: return launch_bm<UQ_INT2, 128>(L, codes, params, x, y, m, stream);
    case UQ_INT4 * 1000 + 32: return launch_bm<UQ_INT4, 32>(L, codes, params, x, y, m, stream);
    case UQ_INT4 * 1000 + 64: return launch_bm<UQ_INT4, 64>(L, codes, params, x, y, m, stream);
    case UQ_INT4 * 1000 + 128: return launch_bm<UQ_INT4, 128>(L, codes, params, x, y, m, stream);
    case UQ_INT8 * 1000 + 64: return launch_bm<UQ_INT8, 64>(L, codes, params, x, y, m, stream);
    case UQ_INT8 * 1000 + 128: return launch_bm<UQ_INT8, 128>(L, codes, params, x, y, m, stream);
    case UQ_NF4 * 1000 + 64: return launch_bm<UQ_NF4, 64>(L, codes, params, x, y, m, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace uq
