// Fused group-wise dequant + GEMM on the bf16 matrix cores, for batched
// decode and prefill ("Ultra LLM Engine", Core Components > Fused Kernels:
// dequantized-weight GEMM during batched decode).
//
// y[m][n] = sum_k bf16(x[m][k]) * bf16(w'[n][k]), fp32 accumulation, where
// w' = fma(q, s, z) (INT-N) or C[q] * a (NF4) is the exact fp32 dequant and
// both casts round to nearest even.
//
// Work split (gfx950):
//   * v_mfma_f32_32x32x16_bf16.  A workgroup is 4 waves and covers BM rows of
//     x by 256 weight rows; wave w owns weight rows [64w, 64w + 64) of the
//     tile (two 32-column MFMA tiles), so every activation fragment read
//     from LDS feeds two MFMAs per M tile.
//   * Weights never pass through LDS: each wave loads its own 64 rows'
//     codes and dequantizes them straight into MFMA B registers, 8 codes per
//     lane per MFMA, exactly once per M tile.
//   * Activations are converted fp16 -> bf16 into a double-buffered LDS
//     tile (BM x 128); the next K step's activation and code loads are in
//     flight while the current one multiplies.
//   * With only ~43 column tiles for a 7B-sized N, K is split across
//     workgroups (so about 256 run at once) and the partial products are
//     added with hardware fp32 atomics into y, which a fill kernel zeroes
//     first; the order of those additions is not fixed, so y can differ from
//     run to run in the last bits when K is split.
//
// Lane layout of one K step of 128: lane l works on row (l % 32) of its
// 32-row tile and on the 64-code half kh = l / 32 of the step; MFMA sub-step
// s (0..7) takes codes [64*kh + 8*s, +8) on both the A and the B side.  (Any
// consistent order of k within an MFMA gives the same dot product.)
#include "device_common.hpp"

namespace uq {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kWN = 64;             // weight rows per wave
constexpr int kBN = kWaves * kWN;   // weight rows per workgroup
constexpr int kBK = 128;            // K per step
constexpr int kLdA = kBK + 8;       // bf16 per LDS row of activations (16-byte pad)

// Raw codes of one lane for one 32-row tile and one K step: 64 consecutive
// codes of one weight row, and the parameters of the groups they span.
template <int S, int G>
struct BRegs {
  static constexpr int bits = Fmt<S>::bits;
  static constexpr int NV = 64 * bits / 128;            // uint4 of codes (1, 2 or 4)
  static constexpr int NGRP = G >= 64 ? 1 : 64 / G;     // groups among the 64 codes
  uint4 code[NV];
  uint32_t par[NGRP];
};

template <int S, int G>
__device__ __forceinline__ void load_b(BRegs<S, G>& b, const uint8_t* __restrict__ codes,
                                       const uint8_t* __restrict__ params, int row, int k0,
                                       int k, size_t rowb, int ng) {
  constexpr int bits = Fmt<S>::bits;
  constexpr int NV = BRegs<S, G>::NV, NGRP = BRegs<S, G>::NGRP;
  const uint8_t* cr = codes + size_t(row) * rowb;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    int kv = k0 + v * (128 / bits);                 // first code of this 16-byte piece
    kv = kv < k ? kv : 0;                           // past K: any valid piece (its x is 0)
    b.code[v] = *reinterpret_cast<const uint4*>(cr + size_t(kv) * bits / 8);
  }
  const int kg = k0 < k ? k0 : 0;
#pragma unroll
  for (int j = 0; j < NGRP; ++j) {
    int g = kg / G + j;
    g = g < ng ? g : ng - 1;  // groups past K (short last step): any valid one (its x is 0)
    const int64_t gi = int64_t(row) * ng + g;
    if constexpr (S == UQ_NF4) b.par[j] = *reinterpret_cast<const uint16_t*>(params + gi * 2);
    else b.par[j] = *reinterpret_cast<const uint32_t*>(params + gi * 4);
  }
}

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Byte i of a dword to fp32 in one instruction.  (Written as shift-and-mask,
// the compiler emits a bit-field extract plus a byte-0 conversion: two.)
template <int I>
__device__ __forceinline__ float ubyte_f32(uint32_t v) {
  float r;
  if constexpr (I == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(v));
  else if constexpr (I == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(v));
  else if constexpr (I == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(v));
  else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(v));
  return r;
}

template <int I>
__device__ __forceinline__ void bytes_to_f32(uint32_t v, float (&f)[4]) {
  f[0] = ubyte_f32<0>(v);
  f[1] = ubyte_f32<1>(v);
  f[2] = ubyte_f32<2>(v);
  f[3] = ubyte_f32<3>(v);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2 v = {__bf16(a), __bf16(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// Dequantize codes [8s, 8s+8) of the lane's 64 to bf16 (exact fp32 dequant,
// then round to nearest even), as an MFMA operand.
template <int S, int G>
__device__ __forceinline__ bf16x8 dequant8(const BRegs<S, G>& b, int s, const float* nf4) {
  constexpr int bits = Fmt<S>::bits;
  float w[8];
  const int grp = G >= 64 ? 0 : (8 * s) / G;
  float sc, zc;
  if constexpr (S == UQ_NF4) {
    sc = h2f(uint16_t(b.par[0]));
    zc = 0.0f;
  } else {
    sc = h2f(uint16_t(b.par[grp] & 0xFFFFu));
    zc = h2f(uint16_t(b.par[grp] >> 16));
  }
  if constexpr (bits == 8) {
    const uint32_t d0 = dword_of(b.code[s >> 1], (s & 1) * 2), d1 = dword_of(b.code[s >> 1], (s & 1) * 2 + 1);
    float q0[4], q1[4];
    bytes_to_f32<0>(d0, q0);
    bytes_to_f32<0>(d1, q1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[i] = __builtin_fmaf(q0[i], sc, zc);
      w[4 + i] = __builtin_fmaf(q1[i], sc, zc);
    }
  } else if constexpr (bits == 4) {
    const uint32_t d = dword_of(b.code[s >> 2], s & 3);
    const uint32_t lo = d & 0x0F0F0F0Fu, hi = (d >> 4) & 0x0F0F0F0Fu;  // codes 0,2,4,6 | 1,3,5,7
    if constexpr (S == UQ_NF4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[2 * i] = nf4[(lo >> (8 * i)) & 0xFu] * sc;
        w[2 * i + 1] = nf4[(hi >> (8 * i)) & 0xFu] * sc;
      }
    } else {
      float qe[4], qo[4];
      bytes_to_f32<0>(lo, qe);
      bytes_to_f32<0>(hi, qo);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[2 * i] = __builtin_fmaf(qe[i], sc, zc);
        w[2 * i + 1] = __builtin_fmaf(qo[i], sc, zc);
      }
    }
  } else {  // 2 bits: codes 8s..8s+7 are 16 bits of one dword
    const uint32_t d = dword_of(b.code[0], s >> 1) >> (16 * (s & 1));
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = __builtin_fmaf(float((d >> (2 * i)) & 3u), sc, zc);
  }
  const uint4 p = make_uint4(pack_bf16(w[0], w[1]), pack_bf16(w[2], w[3]), pack_bf16(w[4], w[5]),
                             pack_bf16(w[6], w[7]));
  return __builtin_bit_cast(bf16x8, p);
}

// Activations: BM rows x 128 columns per K step.  Thread t converts
// PER = BM * 128 / 256 consecutive values of one row.
template <int BM>
struct AStage {
  static constexpr int PER = BM * kBK / kThreads;  // 16, 32 or 64 values
  static constexpr int NV = PER / 8;               // uint4 loads
  uint4 v[NV];
};

template <int BM>
__device__ __forceinline__ void load_a(AStage<BM>& a, const uint16_t* __restrict__ x, int tid, int bm,
                                       int k0, int m, int k) {
  constexpr int PER = AStage<BM>::PER, NV = AStage<BM>::NV;
  constexpr int TPR = kBK / PER;                   // threads per row
  const int r = tid / TPR, c = (tid % TPR) * PER;
  const int row = bm + r < m ? bm + r : m - 1;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    int kv = k0 + c + 8 * v;
    kv = kv < k ? kv : 0;
    a.v[v] = *reinterpret_cast<const uint4*>(x + size_t(row) * size_t(k) + kv);
  }
}

template <int BM>
__device__ __forceinline__ void store_a(const AStage<BM>& a, __bf16* As, int tid, int bm, int k0, int m,
                                        int k) {
  constexpr int PER = AStage<BM>::PER, NV = AStage<BM>::NV;
  constexpr int TPR = kBK / PER;
  const int r = tid / TPR, c = (tid % TPR) * PER;
  const bool live_row = bm + r < m;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const bool live = live_row && k0 + c + 8 * v < k;  // k is a multiple of 32: whole pieces
    uint4 o = make_uint4(0, 0, 0, 0);
    if (live) {
      const uint4 h = a.v[v];
      o.x = pack_bf16(h2f(uint16_t(h.x)), h2f(uint16_t(h.x >> 16)));
      o.y = pack_bf16(h2f(uint16_t(h.y)), h2f(uint16_t(h.y >> 16)));
      o.z = pack_bf16(h2f(uint16_t(h.z)), h2f(uint16_t(h.z >> 16)));
      o.w = pack_bf16(h2f(uint16_t(h.w)), h2f(uint16_t(h.w >> 16)));
    }
    *reinterpret_cast<uint4*>(As + r * kLdA + c + 8 * v) = o;
  }
}

template <int S, int G, int BM>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ params,
                                                        const uint16_t* __restrict__ x,
                                                        float* __restrict__ y, int n, int k, int m,
                                                        int tiles_m, int splits, int steps_per_split) {
  constexpr int TM = BM / 32;  // 32-row MFMA tiles
  __shared__ __attribute__((aligned(16))) __bf16 As[2][BM * kLdA];
  __shared__ float nf4[16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // blockIdx.x: (split, tile_m, tile_n) with the split fastest, so the K
  // pieces of one output tile run side by side
  const int b = blockIdx.x;
  const int split = b % splits, tile = b / splits;
  const int tile_m = tile % tiles_m, tile_n = tile / tiles_m;
  const int bm = tile_m * BM;
  const int steps = (k + kBK - 1) / kBK;
  const int st0 = split * steps_per_split;
  const int st1 = st0 + steps_per_split < steps ? st0 + steps_per_split : steps;
  if (st0 >= st1) return;
  const size_t rowb = size_t(k) * Fmt<S>::bits / 8;
  const int ng = k / G;
  if constexpr (S == UQ_NF4) {
    if (tid < 16) nf4[tid] = nf4_value(tid);
  }

  const int kh = lane >> 5, r32 = lane & 31;
  int brow[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int rr = tile_n * kBN + wave * kWN + t * 32 + r32;
    brow[t] = rr < n ? rr : n - 1;
  }

  f32x16 acc[TM][2];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[a][t][j] = 0.0f;

  // prologue: step st0 into buffer 0
  AStage<BM> an;
  BRegs<S, G> bn[2];
  load_a<BM>(an, x, tid, bm, st0 * kBK, m, k);
#pragma unroll
  for (int t = 0; t < 2; ++t) load_b<S, G>(bn[t], codes, params, brow[t], st0 * kBK + 64 * kh, k, rowb, ng);
  store_a<BM>(an, As[0], tid, bm, st0 * kBK, m, k);
  __syncthreads();

  for (int st = st0; st < st1; ++st) {
    const int buf = (st - st0) & 1;
    BRegs<S, G> bc[2] = {bn[0], bn[1]};
    const bool more = st + 1 < st1;
    if (more) {  // next step's loads in flight during this step's MFMAs
      load_a<BM>(an, x, tid, bm, (st + 1) * kBK, m, k);
#pragma unroll
      for (int t = 0; t < 2; ++t)
        load_b<S, G>(bn[t], codes, params, brow[t], (st + 1) * kBK + 64 * kh, k, rowb, ng);
    }
    // Sub-steps are software-pipelined: while sub-step s's MFMAs run, the
    // wave dequantizes sub-step s+1's weights and reads its activation
    // fragments; the scheduling hints interleave one MFMA with a few VALU
    // instructions so the matrix core and the VALU work at the same time.
    const __bf16* Ab = As[buf];
    bf16x8 bcur[2], acur[TM];
#pragma unroll
    for (int t = 0; t < 2; ++t) bcur[t] = dequant8<S, G>(bc[t], 0, nf4);
#pragma unroll
    for (int a = 0; a < TM; ++a)
      acur[a] = *reinterpret_cast<const bf16x8*>(Ab + (a * 32 + r32) * kLdA + 64 * kh);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16x8 bnxt[2], anxt[TM];
      if (s < 7) {
#pragma unroll
        for (int a = 0; a < TM; ++a)
          anxt[a] = *reinterpret_cast<const bf16x8*>(Ab + (a * 32 + r32) * kLdA + 64 * kh + 8 * (s + 1));
#pragma unroll
        for (int t = 0; t < 2; ++t) bnxt[t] = dequant8<S, G>(bc[t], s + 1, nf4);
      }
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[a][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(acur[a], bcur[t], acc[a][t], 0, 0, 0);
      if (s < 7) {
#pragma unroll
        for (int q = 0; q < 2 * TM; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 48 / (2 * TM), 0); // then some VALU
          if (q < TM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); // and an LDS read
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) bcur[t] = bnxt[t];
#pragma unroll
        for (int a = 0; a < TM; ++a) acur[a] = anxt[a];
      }
    }
    if (more) store_a<BM>(an, As[buf ^ 1], tid, bm, (st + 1) * kBK, m, k);
    __syncthreads();
  }

  // D layout of a 32x32 tile: lane l, element j -> row 8*(j/4) + 4*(l/32) + j%4,
  // column l % 32.
  const bool atomic = splits > 1;
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int col = tile_n * kBN + wave * kWN + t * 32 + r32;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int row = bm + a * 32 + 8 * (j / 4) + 4 * kh + (j % 4);
        if (row < m && col < n) {
          float* dst = y + size_t(row) * size_t(n) + col;
          if (atomic) unsafeAtomicAdd(dst, acc[a][t][j]);
          else *dst = acc[a][t][j];
        }
      }
    }
}

__global__ __launch_bounds__(256) void zero_kernel(float* __restrict__ y, int64_t count) {
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < count; i += stride) y[i] = 0.0f;
}

template <int S, int G, int BM>
hipError_t launch(const uq_layout* L, const void* codes, const void* params, const uint16_t* x,
                  float* y, int m, hipStream_t stream) {
  int n = int(L->n), k = int(L->k);
  int tiles_m = (m + BM - 1) / BM, tiles_n = (n + kBN - 1) / kBN;
  const int tiles = tiles_m * tiles_n;
  const int steps = (k + kBK - 1) / kBK;
  // Split K so that about 256 workgroups (one per CU) share the work.
  int splits = (256 + tiles - 1) / tiles;
  if (splits > steps) splits = steps;
  if (splits < 1) splits = 1;
  int steps_per_split = (steps + splits - 1) / splits;
  splits = (steps + steps_per_split - 1) / steps_per_split;
  if (splits > 1) {
    int64_t count = int64_t(m) * n;
    void* zargs[] = {&y, &count};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&zero_kernel), dim3(1024), dim3(256),
                                         zargs, 0, stream);
    if (e != hipSuccess) return e;
  }
  const uint8_t* c8 = static_cast<const uint8_t*>(codes);
  const uint8_t* p8 = static_cast<const uint8_t*>(params);
  void* args[] = {&c8, &p8, (void*)&x, &y, &n, &k, &m, &tiles_m, &splits, &steps_per_split};
  const dim3 grid(unsigned(tiles * splits)), block(kThreads);
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_kernel<S, G, BM>), grid, block, args, 0, stream);
}

template <int S, int G>
hipError_t launch_bm(const uq_layout* L, const void* codes, const void* params, const uint16_t* x,
                     float* y, int m, hipStream_t stream) {
  if (m <= 32) return launch<S, G, 32>(L, codes, params, x, y, m, stream);
  if (m <= 64) return launch<S, G, 64>(L, codes, params, x, y, m, stream);
  return launch<S, G, 128>(L, codes, params, x, y, m, stream);
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
