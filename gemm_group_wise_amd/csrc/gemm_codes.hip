// Fused group-wise dequant + GEMM on the bf16 matrix cores that multiplies
// the integer codes themselves: INT2 / INT4 / INT8 layouts whose groups hold
// 64 or 128 codes ("Ultra LLM Engine", Core Components > Fused Kernels:
// dequantized-weight GEMM during batched decode; Highlights, Batching).
//
//   y[m][n] = sum_g ( s[n][g] * T[m][n][g] + z[n][g] * X[m][g] ),
//   T = sum_{k in g} q[n][k] * bf16(x[m][k]),   X = sum_{k in g} bf16(x[m][k]),
//
// which is bf16(x) . w'^T with the weights unrounded (w' = q s + z).  Only x
// is cast to bf16 (round to nearest even); the codes are exact in bf16:
// INT4 / INT2 codes as 128 + q (bf16 0x4300 | q: one v_and_or_b32 per pair of
// codes after a shift), INT8 codes as q (byte -> fp32 -> bf16, exact below 256).
// Per group, each 16 x 16 output tile runs a chain of G / 32
// v_mfma_f32_16x16x32_bf16 that starts from C = -128 X (0 for INT8) and so
// ends at T; then y += s T + z X in fp32 (two v_fma_f32 per output).  For
// x = e_k this gives fma(s, q, z) = w' exactly.
//
// Why this form: scaling once per group costs about 64 / G VALU cycles per
// MFMA cycle and unpacking a code about 28 / BM, against about 93 / BM for
// dequantizing every weight to bf16 once per row tile; at M <= 64 the GEMM is
// bound by exactly that VALU work.
//
// MFMA lane layout (16x16x32): lane l holds A[row l % 16][k-block l / 16] (8
// consecutive k), B[k-block l / 16][column l % 16] and D[rows 4 (l / 16) + i]
// [column l % 16].  Rows are activation rows, columns weight rows.  Within a
// group the k order is free as long as A and B agree: lane k-block kb of
// every MFMA of a group's chain takes the kb-th run of 8 * G / 32 consecutive
// codes of the group (one LDS read per lane and group), in the order the
// unpacking produces them, and the activations are staged in that order.
//
// Work split: a workgroup of four waves owns BM = 16 TM WM activation rows by
// BN = 16 TN WN weight rows; wave (wm, wn) keeps TM x TN output tiles (the
// chain accumulators and y).  K is walked in steps of 128: each step's
// activations (fp16 -> bf16, with the per-group sums X), codes and group
// parameters go global -> registers (PD steps ahead) -> LDS, once per
// workgroup; then every wave computes the step.  The K steps of a tile may be
// split over up to kGemmMaxSplit workgroups (partial tiles summed in split
// order by the last to arrive, as in the dequantizing GEMM).
#include <atomic>

#include "device_common.hpp"

namespace uq {
namespace {

typedef __bf16 bf16x8c __attribute__((ext_vector_type(8)));
typedef float f32x4c __attribute__((ext_vector_type(4)));

constexpr int kCKS = 128;              // k per step
constexpr int kCThreads = 256;         // four waves
constexpr int kCXPitch = kCKS * 2 + 16;  // LDS bytes per staged activation row (16-byte pad)

template <int S> constexpr int code_base() { return S == UQ_INT8 ? 0 : 128; }

// Where position t (0..15) of a 16-activation chunk goes: MFMA dj (0 or 1)
// after the chunk's first, element e (0..7).  It mirrors the element order of
// the unpacked codes (see unpack_b).
template <int S>
__device__ __forceinline__ constexpr int chunk_dj(int t) {
  if constexpr (S == UQ_INT2) return (t >> 2) & 1;
  else return t >> 3;
}
template <int S>
__device__ __forceinline__ constexpr int chunk_e(int t) {
  if constexpr (S == UQ_INT4) {
    constexpr int inv[8] = {0, 2, 4, 6, 1, 3, 5, 7};  // element of run position t % 8
    return inv[t & 7];
  } else if constexpr (S == UQ_INT2) {
    return 2 * (t & 3) + (t >> 3);
  } else {
    return t & 7;
  }
}

// Position (0..15) in a 16-activation chunk of element e of MFMA dj: the
// inverse of (chunk_dj, chunk_e).
template <int S>
__device__ __forceinline__ constexpr int chunk_src(int dj, int e) {
  int r = 0;
  for (int t = 0; t < 16; ++t)
    if (chunk_dj<S>(t) == dj && chunk_e<S>(t) == e) r = t;
  return r;
}

// B operand of MFMA j of a chain from the lane's run of codes (dwords).
//   INT4: dword j = codes 8j..8j+7; pairs (c_i, c_i+4), i = 0..3.
//   INT2: dword j / 2 = 16 codes; MFMA j takes pairs (c_i, c_i+8) for
//         i = 4 (j % 2) .. + 3.
//   INT8: dwords 2j, 2j + 1 = codes 8j..8j+7 in order.
template <int S, int RW>
__device__ __forceinline__ bf16x8c unpack_b(const uint32_t (&run)[RW], int j) {
  uint4 v;
  if constexpr (S == UQ_INT4) {
    const uint32_t d = run[j];
    constexpr uint32_t mg = 0x43004300u;
    v.x = and_or(d, 0x000F000Fu, mg);
    v.y = and_or(d >> 4, 0x000F000Fu, mg);
    v.z = and_or(d >> 8, 0x000F000Fu, mg);
    v.w = and_or(d >> 12, 0x000F000Fu, mg);
  } else if constexpr (S == UQ_INT2) {
    const uint32_t d = run[j >> 1] >> (8 * (j & 1));
    constexpr uint32_t mg = 0x43004300u;
    v.x = and_or(d, 0x00030003u, mg);
    v.y = and_or(d >> 2, 0x00030003u, mg);
    v.z = and_or(d >> 4, 0x00030003u, mg);
    v.w = and_or(d >> 6, 0x00030003u, mg);
  } else {
    const uint32_t d0 = run[2 * j], d1 = run[2 * j + 1];
    auto pk = [](float a, float b) {
      const bf16x2 p = {__bf16(a), __bf16(b)};  // exact: integers below 256
      return __builtin_bit_cast(uint32_t, p);
    };
    v.x = pk(float(d0 & 0xFFu), float((d0 >> 8) & 0xFFu));
    v.y = pk(float((d0 >> 16) & 0xFFu), float(d0 >> 24));
    v.z = pk(float(d1 & 0xFFu), float((d1 >> 8) & 0xFFu));
    v.w = pk(float((d1 >> 16) & 0xFFu), float(d1 >> 24));
  }
  return __builtin_bit_cast(bf16x8c, v);
}

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ uint32_t bf16_pair(uint32_t h2) {
  const bf16x2 p = {__bf16(h2f(uint16_t(h2 & 0xFFFFu))), __bf16(h2f(uint16_t(h2 >> 16)))};
  return __builtin_bit_cast(uint32_t, p);
}

// Workgroup barrier for LDS only: this wave's LDS accesses complete
// (lgkmcnt(0)), then s_barrier.  __syncthreads() also fences global memory,
// which on gfx9 means waiting for every outstanding vector-memory load --
// including the prefetches of later steps this kernel keeps in flight.  The
// empty asm statements stop the compiler from moving LDS accesses across.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), gfx9 encoding
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---- More than 64 activation rows: activations prepared once ----
//
// x_chain_kernel turns x into bf16 in the chain order with the per-group
// sums (X, -128 X), once per call, into the caller's workspace; the tile
// kernel then copies activation tiles without touching them.  (Converting
// in every workgroup cost about half of the tile kernel's VALU work at
// M = 256: each activation is read by N / BN workgroups.)

// One thread per 16 activations: bf16 in chain order (two 16-byte blocks),
// and the group's sums reduced over its G / 16 consecutive lanes by DPP.
template <int S, int G>
__global__ __launch_bounds__(256) void x_chain_kernel(const uint16_t* __restrict__ x, uint16_t* __restrict__ xc,
                                                      float2* __restrict__ xt, int m, int k) {
  constexpr int CL = G / 32;
  const int64_t it = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int cpr = k / 16;
  const int64_t total = int64_t(m) * cpr;
  const int64_t itc = it < total ? it : total - 1;  // past the end: a repeat, not written
  const int row = int(itc / cpr), c = int(itc % cpr);
  const int g = c / (G / 16), cg = c % (G / 16);
  const int kbs = 16 * cg / (8 * CL), jb = (16 * cg % (8 * CL)) / 8;
  const uint4* src = reinterpret_cast<const uint4*>(x + size_t(row) * size_t(k) + 16 * c);
  const uint4 v0 = src[0], v1 = src[1];
  float f[16];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t d = dword_of(t < 4 ? v0 : v1, t & 3);
    f[2 * t] = h2f(uint16_t(d & 0xFFFFu));
    f[2 * t + 1] = h2f(uint16_t(d >> 16));
  }
  const bf16x2 one2 = {__bf16(1.0f), __bf16(1.0f)};
  float sx = 0.0f;
  uint4 o[2];
#pragma unroll
  for (int dj = 0; dj < 2; ++dj) {
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const bf16x2 v = {__bf16(f[chunk_src<S>(dj, 2 * p)]), __bf16(f[chunk_src<S>(dj, 2 * p + 1)])};
      w[p] = __builtin_bit_cast(uint32_t, v);
      sx = __builtin_amdgcn_fdot2_f32_bf16(v, one2, sx, false);
    }
    o[dj] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  sx += dpp_mov<0xB1>(sx);   // quad_perm [1,0,3,2]
  sx += dpp_mov<0x4E>(sx);   // quad_perm [2,3,0,1]
  if constexpr (G == 128) sx += dpp_mov<0x141>(sx);  // row_half_mirror
  if (it < total) {
    uint16_t* dst = xc + size_t(row) * size_t(k) + g * G + 8 * kbs;
    *reinterpret_cast<uint4*>(dst + 32 * jb) = o[0];
    *reinterpret_cast<uint4*>(dst + 32 * (jb + 1)) = o[1];
    if (cg == 0) xt[size_t(row) * size_t(k / G) + g] = make_float2(sx, float(-code_base<S>()) * sx);
  }
}

constexpr int kCPW = 32;  // groups per parameter window of the tile kernel

template <int S, int G, int TM, int TN, int WM>
struct CGeo {
  static constexpr int WN = 4 / WM;
  static constexpr int BM = 16 * TM * WM, BN = 16 * TN * WN;
  static constexpr int bits = Fmt<S>::bits;
  static constexpr int CL = G / 32;                  // MFMAs per group
  static constexpr int GPS = kCKS / G;               // groups per step
  static constexpr int RB = kCKS * bits / 8;         // code bytes per row per step
  static constexpr int CPITCH = RB + 16;             // their LDS pitch
  static constexpr int RUNB = CL * 8 * bits / 8;     // bytes of a lane's run (one group)
  static constexpr int RW = RUNB / 4;                // its dwords
  static constexpr int XQ = BM * 16 / kCThreads;     // 16-byte activation pieces per thread per step
  static constexpr int CP = BN * RB / 16;            // 16-byte code pieces per step
  static constexpr int CPT = (CP + kCThreads - 1) / kCThreads;
  static constexpr int TT = BM * GPS;                // (X, -128 X) pairs per step
  static constexpr int PWT = BN * kCPW / kCThreads;  // parameter dwords per thread per window
  static_assert(TT <= kCThreads && XQ >= 1 && (BN * kCPW) % kCThreads == 0, "step geometry");
  static_assert(G == 64 || G == 128, "groups of 64 or 128 codes");
  static_assert(RUNB % 4 == 0 && RB % 16 == 0, "run and step geometry");
};

template <int S, int G, int TM, int TN, int WM>
struct Prefetch {
  using Ge = CGeo<S, G, TM, TN, WM>;
  uint4 xv[Ge::XQ];
  uint4 cv[Ge::CPT];
  float2 tv;
};

// The tile kernel: four waves, BM = 16 TM WM activation rows by BN = 16 TN WN
// weight rows; wave (wm, wn) keeps TM x TN output tiles.  K is walked in
// steps of 128 whose activation tile, (X, -128 X) pairs and codes go global
// -> registers (one step ahead) -> LDS; the group parameters of a window of
// kCPW groups are loaded (consecutive lanes, consecutive groups of a row)
// into LDS at the start of the window.
template <int S, int G, int TM, int TN, int WM>
__global__ __launch_bounds__(kCThreads, 2) void gemm_codes_kernel(const uint8_t* __restrict__ codes,
                                                               const uint8_t* __restrict__ params,
                                                               const uint16_t* __restrict__ xc,
                                                               const float2* __restrict__ xt, float* __restrict__ y,
                                                               int n, int k, int m, int tiles_m) {
  using Ge = CGeo<S, G, TM, TN, WM>;
  using Pre = Prefetch<S, G, TM, TN, WM>;
  constexpr int bits = Ge::bits, CL = Ge::CL, GPS = Ge::GPS, BM = Ge::BM, BN = Ge::BN;
  __shared__ __attribute__((aligned(16))) uint8_t xs[BM * kCXPitch];
  __shared__ __attribute__((aligned(16))) float xsum[GPS * BM];
  __shared__ __attribute__((aligned(16))) float xneg[GPS * BM];
  __shared__ __attribute__((aligned(16))) uint8_t cs[BN * Ge::CPITCH];
  __shared__ __attribute__((aligned(16))) uint32_t ps[BN * kCPW];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / Ge::WN, wn = wave % Ge::WN;
  const int tile = blockIdx.x;
  const int tile_m = tile % tiles_m, tile_n = tile / tiles_m;
  const int bm = tile_m * BM, bn = tile_n * BN;
  const int rowb = k * bits / 8;
  const int ng = k / G;
  const int steps = (k + kCKS - 1) / kCKS;

  // ---- global -> registers for step st (clamped: rows past M or N, k past K) ----
  auto prefetch = [&](Pre& p, int st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < Ge::XQ; ++i) {
      const int q = i * kCThreads + tid;
      const int row = q / 16, c = q % 16;
      int mr = bm + row;
      mr = mr < m ? mr : m - 1;
      p.xv[i] = *reinterpret_cast<const uint4*>(xc + size_t(mr) * size_t(k) + st * kCKS + 8 * c);
    }
#pragma unroll
    for (int j = 0; j < Ge::CPT; ++j) {
      const int q0 = j * kCThreads + tid;
      const int q = q0 < Ge::CP ? q0 : Ge::CP - 1;
      const int row = q / (Ge::RB / 16), pc = q % (Ge::RB / 16);
      int gr = bn + row;
      gr = gr < n ? gr : n - 1;
      p.cv[j] = load_stream<uint4>(codes + size_t(gr) * size_t(rowb) + st * Ge::RB + 16 * pc);
    }
    {
      const int q = tid < Ge::TT ? tid : Ge::TT - 1;
      int mr = bm + q / GPS;
      mr = mr < m ? mr : m - 1;
      int gg = st * GPS + q % GPS;
      gg = gg < ng ? gg : ng - 1;
      p.tv = xt[size_t(mr) * size_t(ng) + gg];
    }
  };
  auto stage = [&](const Pre& p) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < Ge::XQ; ++i) {
      const int q = i * kCThreads + tid;
      *reinterpret_cast<uint4*>(xs + (q / 16) * kCXPitch + 16 * (q % 16)) = p.xv[i];
    }
#pragma unroll
    for (int j = 0; j < Ge::CPT; ++j) {
      const int q0 = j * kCThreads + tid;
      if (q0 < Ge::CP) *reinterpret_cast<uint4*>(cs + (q0 / (Ge::RB / 16)) * Ge::CPITCH + 16 * (q0 % (Ge::RB / 16))) = p.cv[j];
    }
    if (tid < Ge::TT) {
      xsum[(tid % GPS) * BM + tid / GPS] = p.tv.x;
      xneg[(tid % GPS) * BM + tid / GPS] = p.tv.y;
    }
  };

  const int l16 = lane & 15, kb = lane >> 4;
  f32x4c yacc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int t = 0; t < TN; ++t) yacc[a][t] = f32x4c{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](int st, int w0) __attribute__((always_inline)) {
    const int gvalid = (k - st * kCKS) / G < GPS ? (k - st * kCKS) / G : GPS;
#pragma unroll
    for (int g = 0; g < GPS; ++g) {
      if (g >= gvalid) break;  // uniform: the last step of an odd number of 64-code groups
      uint32_t run[TN][Ge::RW];
      float sc[TN], zc[TN];
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const int r = 16 * (TN * wn + t) + l16;
        const uint8_t* src = cs + r * Ge::CPITCH + g * (G * bits / 8) + kb * Ge::RUNB;
        if constexpr (Ge::RW == 1) {
          run[t][0] = *reinterpret_cast<const uint32_t*>(src);
        } else if constexpr (Ge::RW == 2) {
          const uint2 v = *reinterpret_cast<const uint2*>(src);
          run[t][0] = v.x; run[t][1] = v.y;
        } else {
#pragma unroll
          for (int q = 0; q < Ge::RW / 4; ++q) {
            const uint4 v = reinterpret_cast<const uint4*>(src)[q];
            run[t][4 * q] = v.x; run[t][4 * q + 1] = v.y; run[t][4 * q + 2] = v.z; run[t][4 * q + 3] = v.w;
          }
        }
        const uint32_t pw = ps[r * kCPW + st * GPS + g - w0];
        sc[t] = h2f(uint16_t(pw & 0xFFFFu));
        zc[t] = h2f(uint16_t(pw >> 16));
      }
      f32x4c xsv[TM], acc[TM][TN];
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        const int r0 = 16 * (TM * wm + a) + 4 * kb;
        xsv[a] = *reinterpret_cast<const f32x4c*>(xsum + g * BM + r0);
        const f32x4c c0 = *reinterpret_cast<const f32x4c*>(xneg + g * BM + r0);
#pragma unroll
        for (int t = 0; t < TN; ++t) acc[a][t] = c0;  // the chain starts at -128 X (0 for INT8)
      }
#pragma unroll
      for (int j = 0; j < CL; ++j) {
        bf16x8c av[TM], bv[TN];
#pragma unroll
        for (int a = 0; a < TM; ++a)
          av[a] = *reinterpret_cast<const bf16x8c*>(xs + (16 * (TM * wm + a) + l16) * kCXPitch +
                                                    (g * G + 32 * j + 8 * kb) * 2);
#pragma unroll
        for (int t = 0; t < TN; ++t) bv[t] = unpack_b<S, Ge::RW>(run[t], j);
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
          for (int t = 0; t < TN; ++t) acc[a][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[a], bv[t], acc[a][t], 0, 0, 0);
      }
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            yacc[a][t][i] = __builtin_fmaf(sc[t], acc[a][t][i], yacc[a][t][i]);
            yacc[a][t][i] = __builtin_fmaf(zc[t], xsv[a][i], yacc[a][t][i]);
          }
    }
  };

  // Parameter windows of kCPW groups; within a window the K steps run with
  // the next step's loads in flight during each step's products.
  for (int w0 = 0; w0 < ng; w0 += kCPW) {
    const int sw0 = w0 / GPS, sw1 = (w0 + kCPW < ng ? w0 + kCPW : ng + GPS - 1) / GPS;  // the window's steps
    uint32_t pv[Ge::PWT];
#pragma unroll
    for (int i = 0; i < Ge::PWT; ++i) {
      const int q = i * kCThreads + tid;
      int gr = bn + q / kCPW, gg = w0 + q % kCPW;
      gr = gr < n ? gr : n - 1;
      gg = gg < ng ? gg : ng - 1;
      pv[i] = load_stream<uint32_t>(params + (size_t(gr) * size_t(ng) + gg) * 4);
    }
    Pre pre;
    prefetch(pre, sw0);
    lds_barrier();  // the previous window's products are done with the LDS
#pragma unroll
    for (int i = 0; i < Ge::PWT; ++i) ps[i * kCThreads + tid] = pv[i];
    for (int st = sw0; st < sw1; ++st) {
      lds_barrier();  // every wave is done with the previous step's LDS
      stage(pre);
      lds_barrier();
      prefetch(pre, st + 1 < sw1 ? st + 1 : st);  // the last step repeats its loads (not staged)
      compute(st, w0);
    }
  }
  (void)steps;

  // D layout: lane l, element i -> activation row 4 (l / 16) + i, weight row l % 16 of its tile.
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const int col = bn + 16 * (TN * wn + t) + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = bm + 16 * (TM * wm + a) + 4 * kb + i;
        if (row < m && col < n) y[size_t(row) * size_t(n) + col] = yacc[a][t][i];
      }
    }
}

// ---- Up to 64 activation rows: codes streamed straight into registers ----
//
// Up to 64 rows the GEMM is bound by memory traffic and latency, not by the
// matrix cores.  A workgroup of W waves owns 16 W weight rows (16 per wave)
// and a K range (the K split); per block of XB activations of that range it
//   * issues the loads of the block's activations and of its rows' group
//     parameters (consecutive lanes, consecutive groups of a row), then every
//     code of the wave's 16 rows that the block needs, directly in the MFMA
//     layout (lane l: weight row l % 16, k-block l / 16's run of each group:
//     one wave instruction reads 16 rows x the group's bytes),
//   * stages the activations in LDS (bf16, packed straight into the chain
//     order, with the per-group sums X and -128 X reduced across lanes by
//     DPP) and the parameters,
//   * synchronises once and runs every group's chain and scaling.
// No workgroup barrier sits between a block's loads and its products.
template <int S, int G, int TM, int W>
struct SGeo {
  static constexpr int BM = 16 * TM, BN = 16 * W, NT = 64 * W;
  static constexpr int bits = Fmt<S>::bits;
  static constexpr int CL = G / 32;
  static constexpr int XB = 16384 / BM;               // activations per row per block (32 KB of bf16)
  static constexpr int NGB = XB / G;                  // groups per block
  static constexpr int RUNB = CL * 8 * bits / 8;      // bytes of a lane's run of one group
  static constexpr int RW = RUNB / 4;
  static constexpr int XPITCH = XB * 2 + 16;
  static constexpr int CPR = XB / 16;                 // 16-activation chunks per row per block
  static constexpr int XI = BM * CPR;
  static constexpr int XPT = XI / NT;                 // chunks staged per thread
  static constexpr int PB = BN * NGB;                 // parameter dwords per block
  static constexpr int PPT = (PB + NT - 1) / NT;
  static_assert(XI % NT == 0 && CPR % 8 == 0 && NGB >= 1, "staging geometry");
};

template <int S, int G, int TM, int W>
__global__ __launch_bounds__(64 * W) void gemm_codes_stream_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ params, const uint16_t* __restrict__ x,
    float* __restrict__ y, int n, int k, int m, int tiles_m, int ksplit, float* __restrict__ part,
    unsigned* __restrict__ arrivals) {
  using Ge = SGeo<S, G, TM, W>;
  constexpr int bits = Ge::bits, CL = Ge::CL, BM = Ge::BM, BN = Ge::BN, NGB = Ge::NGB, RW = Ge::RW, NT = Ge::NT;
  __shared__ __attribute__((aligned(16))) uint8_t xs[BM * Ge::XPITCH];
  __shared__ __attribute__((aligned(16))) float xsum[NGB * BM];
  __shared__ __attribute__((aligned(16))) float xneg[NGB * BM];
  __shared__ __attribute__((aligned(16))) uint32_t ps[Ge::PB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x;
  const int split = b % ksplit, tile = b / ksplit;
  const int tile_m = tile % tiles_m, tile_n = tile / tiles_m;
  const int bm = tile_m * BM, bn = tile_n * BN;
  const int ng = k / G;
  const int g0 = split * ng / ksplit, g1 = (split + 1) * ng / ksplit;  // this workgroup's groups
  const int rowb = k * bits / 8;
  const int l16 = lane & 15, kb = lane >> 4;
  int wr = bn + 16 * wave + l16;
  wr = wr < n ? wr : n - 1;  // rows past N: computed, not stored
  const uint8_t* crow = codes + size_t(wr) * size_t(rowb) + kb * Ge::RUNB;

  f32x4c yacc[TM];
#pragma unroll
  for (int a = 0; a < TM; ++a) yacc[a] = f32x4c{0.0f, 0.0f, 0.0f, 0.0f};

  // Registers: the block's activations and parameters (until staged) and its codes.
  uint4 xv[Ge::XPT][2];
  uint32_t pv[Ge::PPT];
  uint32_t run[1][NGB][RW];

  // (1) loads of block gb: activations and parameters for staging, then the
  //     lane's code runs (clamped: rows past M or N, groups past the range)
  auto load_block = [&](int gb, uint32_t (&rr)[NGB][RW]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < Ge::XPT; ++i) {
      const int it = i * NT + tid;
      const int row = it / Ge::CPR, c = it % Ge::CPR;
      int mr = bm + row;
      mr = mr < m ? mr : m - 1;
      int kk = gb * G + 16 * c;
      kk = kk < k ? kk : k - 16;
      const uint4* src = reinterpret_cast<const uint4*>(x + size_t(mr) * size_t(k) + kk);
      xv[i][0] = src[0];
      xv[i][1] = src[1];
    }
#pragma unroll
    for (int i = 0; i < Ge::PPT; ++i) {
      int q = i * NT + tid;
      q = q < Ge::PB ? q : Ge::PB - 1;
      int pr = bn + q / NGB, gg = gb + q % NGB;
      pr = pr < n ? pr : n - 1;
      gg = gg < g1 ? gg : g1 - 1;
      pv[i] = load_stream<uint32_t>(params + (size_t(pr) * size_t(ng) + gg) * 4);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < NGB; ++g) {
      const int gg = gb + g < g1 ? gb + g : g1 - 1;
      const uint8_t* src = crow + size_t(gg) * (G * bits / 8);
      if constexpr (RW == 1) {
        rr[g][0] = load_stream<uint32_t>(src);
      } else if constexpr (RW == 2) {
        const uint2 v = load_stream<uint2>(src);
        rr[g][0] = v.x; rr[g][1] = v.y;
      } else {
#pragma unroll
        for (int q = 0; q < RW / 4; ++q) {
          const uint4 v = load_stream<uint4>(src + 16 * q);
          rr[g][4 * q] = v.x; rr[g][4 * q + 1] = v.y; rr[g][4 * q + 2] = v.z; rr[g][4 * q + 3] = v.w;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // (2) stage the loaded activations (bf16 packed in chain order, group sums
  //     by DPP) and parameters into LDS
  auto stage_block = [&]() __attribute__((always_inline)) {
    lds_barrier();  // the previous block's products are done with the LDS
#pragma unroll
    for (int i = 0; i < Ge::XPT; ++i) {
      const int it = i * NT + tid;
      const int row = it / Ge::CPR, c = it % Ge::CPR;
      const int g = c / (G / 16), cg = c % (G / 16);
      const int kbs = 16 * cg / (8 * CL), jb = (16 * cg % (8 * CL)) / 8;
      float f[16];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t d = dword_of(xv[i][t >> 2], t & 3);
        f[2 * t] = h2f(uint16_t(d & 0xFFFFu));
        f[2 * t + 1] = h2f(uint16_t(d >> 16));
      }
      const bf16x2 one2 = {__bf16(1.0f), __bf16(1.0f)};
      float sx = 0.0f;
      uint8_t* dst = xs + row * Ge::XPITCH + (g * G + 8 * kbs) * 2;
#pragma unroll
      for (int dj = 0; dj < 2; ++dj) {
        uint32_t o[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const bf16x2 v = {__bf16(f[chunk_src<S>(dj, 2 * p)]), __bf16(f[chunk_src<S>(dj, 2 * p + 1)])};
          o[p] = __builtin_bit_cast(uint32_t, v);
          sx = __builtin_amdgcn_fdot2_f32_bf16(v, one2, sx, false);
        }
        *reinterpret_cast<uint4*>(dst + 32 * (jb + dj) * 2) = make_uint4(o[0], o[1], o[2], o[3]);
      }
      // sum over the G / 16 lanes of the (row, group): quads, then half-row mirror (every lane gets the total)
      sx += dpp_mov<0xB1>(sx);   // quad_perm [1,0,3,2]
      sx += dpp_mov<0x4E>(sx);   // quad_perm [2,3,0,1]
      if constexpr (G == 128) sx += dpp_mov<0x141>(sx);  // row_half_mirror
      if (cg == 0) {
        xsum[g * BM + row] = sx;
        xneg[g * BM + row] = float(-code_base<S>()) * sx;
      }
    }
#pragma unroll
    for (int i = 0; i < Ge::PPT; ++i) {
      const int q = i * NT + tid;
      if (q < Ge::PB) ps[q] = pv[i];
    }
    lds_barrier();
  };

  // (3) every group's chain and scaling for block gb
  auto compute_block = [&](int gb, const uint32_t (&rr)[NGB][RW]) __attribute__((always_inline)) {
    const int nvalid = g1 - gb < NGB ? g1 - gb : NGB;  // groups of this block (uniform)
    const uint32_t* prw = ps + (16 * wave + l16) * NGB;
#pragma unroll
    for (int g = 0; g < NGB; ++g) {
      if (g >= nvalid) break;  // uniform
      const uint32_t pw = prw[g];
      const float sc = h2f(uint16_t(pw & 0xFFFFu)), zc = h2f(uint16_t(pw >> 16));
      f32x4c xsv[TM], acc[TM];
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        xsv[a] = *reinterpret_cast<const f32x4c*>(xsum + g * BM + 16 * a + 4 * kb);
        acc[a] = *reinterpret_cast<const f32x4c*>(xneg + g * BM + 16 * a + 4 * kb);
      }
#pragma unroll
      for (int j = 0; j < CL; ++j) {
        const bf16x8c bv = unpack_b<S, RW>(rr[g], j);
#pragma unroll
        for (int a = 0; a < TM; ++a) {
          const bf16x8c av = *reinterpret_cast<const bf16x8c*>(xs + (16 * a + l16) * Ge::XPITCH +
                                                               (g * G + 32 * j + 8 * kb) * 2);
          acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[a], 0, 0, 0);
        }
      }
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          yacc[a][i] = __builtin_fmaf(sc, acc[a][i], yacc[a][i]);
          yacc[a][i] = __builtin_fmaf(zc, xsv[a][i], yacc[a][i]);
        }
    }
  };

  // Block by block: every load of the block at once, then stage, then the
  // products.  (Issuing the next block's code loads before the products of
  // this one took more registers than it saved: one block ahead measured
  // 15.0 against 12.4 us at M = 16 and no better at M = 32 or 64.)
  for (int gb = g0; gb < g1; gb += NGB) {
    load_block(gb, run[0]);
    stage_block();
    compute_block(gb, run[0]);
  }

  // D layout: lane l, element i -> activation row 4 (l / 16) + i of tile a, weight row l % 16 of the wave.
  const int col = bn + 16 * wave + l16;
  if (ksplit > 1) {
    // K split: partial tiles with agent-scope atomic stores, one arrival
    // counter per tile, the last workgroup adds the partial tiles in split
    // order (as in the step kernel below).
    const size_t rows = size_t(tiles_m) * BM;
    float* dst = part + size_t(split) * rows * size_t(n);
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (col < n)
          __hip_atomic_store(dst + size_t(bm + 16 * a + 4 * kb + i) * size_t(n) + col, yacc[a][i], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the partial tile has been written
    __syncthreads();
    __shared__ unsigned last;
    if (tid == 0) {
      const unsigned before = atomicAdd(arrivals + tile, 1u);
      last = before == unsigned(ksplit - 1);
      if (last) atomicExch(arrivals + tile, 0u);
    }
    __syncthreads();
    if (!last) return;
    constexpr int E = BM * BN / NT;
    float v[kGemmMaxSplit][E];
#pragma unroll
    for (int sp = 0; sp < kGemmMaxSplit; ++sp) {
      const int spc = sp < ksplit ? sp : ksplit - 1;
      const float* src = part + (size_t(spc) * rows + size_t(bm)) * size_t(n);
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const int e = i * NT + tid;
        const int c = min(bn + e % BN, n - 1);
        v[sp][i] = __hip_atomic_load(src + size_t(e / BN) * size_t(n) + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
#pragma unroll
    for (int i = 0; i < E; ++i) {
      float sum = v[0][i];
#pragma unroll
      for (int sp = 1; sp < kGemmMaxSplit; ++sp) sum = sp < ksplit ? sum + v[sp][i] : sum;
      const int e = i * NT + tid;
      const int row = bm + e / BN, c = bn + e % BN;
      if (row < m && c < n) y[size_t(row) * size_t(n) + c] = sum;
    }
    return;
  }
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = bm + 16 * a + 4 * kb + i;
      if (row < m && col < n) y[size_t(row) * size_t(n) + col] = yacc[a][i];
    }
}

template <int S, int G, int TM, int W>
hipError_t launch_stream_t(const uq_layout* L, const void* codes, const void* params, const uint16_t* x, float* y,
                           int m, float* part, unsigned* arrivals, int cus, hipStream_t stream) {
  using Ge = SGeo<S, G, TM, W>;
  int n = int(L->n), k = int(L->k);
  int tiles_m = (m + Ge::BM - 1) / Ge::BM;
  const int64_t tiles = int64_t(tiles_m) * ((int64_t(n) + Ge::BN - 1) / Ge::BN);
  int ksplit = 1;
  if (tiles <= kGemmMaxSplitTiles) {
    static std::atomic<int> cached{0};
    int occ = cached.load(std::memory_order_relaxed);
    if (occ <= 0) {
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
              &occ, reinterpret_cast<const void*>(&gemm_codes_stream_kernel<S, G, TM, W>), Ge::NT, 0) != hipSuccess ||
          occ < 1)
        occ = 1;
      cached.store(occ, std::memory_order_relaxed);
    }
    const int ng = k / G;
    int64_t ks = int64_t(cus) * occ / tiles;
    if (ks > kGemmMaxSplit) ks = kGemmMaxSplit;
    if (ks > ng / 2) ks = ng / 2;
    ksplit = ks > 1 ? int(ks) : 1;
  }
  const int64_t nb = tiles * ksplit;
  if (nb > 0x7fffffff) return hipErrorInvalidValue;
  const uint8_t* c8 = static_cast<const uint8_t*>(codes);
  const uint8_t* p8 = static_cast<const uint8_t*>(params);
  void* args[] = {&c8, &p8, (void*)&x, &y, &n, &k, &m, &tiles_m, &ksplit, &part, &arrivals};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_codes_stream_kernel<S, G, TM, W>), dim3(unsigned(nb)),
                         dim3(Ge::NT), args, 0, stream);
}

template <int S, int G, int TM, int TN, int WM>
hipError_t launch_codes_t(const uq_layout* L, const void* codes, const void* params, const uint16_t* x, float* y,
                          int m, uint16_t* xc, float2* xt, hipStream_t stream) {
  using Ge = CGeo<S, G, TM, TN, WM>;
  int n = int(L->n), k = int(L->k);
  {  // activations to bf16 in chain order, with the group sums
    const int64_t chunks = int64_t(m) * (k / 16);
    const int64_t blocks = (chunks + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    int mm = m, kk = k;
    void* args[] = {(void*)&x, &xc, &xt, &mm, &kk};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&x_chain_kernel<S, G>), dim3(unsigned(blocks)),
                                         dim3(256), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  int tiles_m = (m + Ge::BM - 1) / Ge::BM;
  const int64_t nb = int64_t(tiles_m) * ((int64_t(n) + Ge::BN - 1) / Ge::BN);
  if (nb > 0x7fffffff) return hipErrorInvalidValue;
  const uint8_t* c8 = static_cast<const uint8_t*>(codes);
  const uint8_t* p8 = static_cast<const uint8_t*>(params);
  const uint16_t* xcc = xc;
  const float2* xtc = xt;
  void* args[] = {&c8, &p8, &xcc, &xtc, &y, &n, &k, &m, &tiles_m};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_codes_kernel<S, G, TM, TN, WM>), dim3(unsigned(nb)),
                         dim3(kCThreads), args, 0, stream);
}

template <int S, int G>
hipError_t launch_codes_m(const CodesPlan& p, const uq_layout* L, const void* codes, const void* params,
                          const uint16_t* x, float* y, int m, float* part, unsigned* arrivals, uint16_t* xc,
                          float2* xt, int cus, hipStream_t stream) {
  switch (p.cfg) {
    case 0: return launch_stream_t<S, G, 1, 4>(L, codes, params, x, y, m, part, arrivals, cus, stream);
    case 1: return launch_stream_t<S, G, 2, 4>(L, codes, params, x, y, m, part, arrivals, cus, stream);
    case 2: return launch_stream_t<S, G, 4, 4>(L, codes, params, x, y, m, part, arrivals, cus, stream);
    default: return launch_codes_t<S, G, 4, 4, 2>(L, codes, params, x, y, m, xc, xt, stream);
  }
}

}  // namespace

hipError_t launch_gemm_codes(const uq_layout* L, const void* codes, const void* params, const uint16_t* x, float* y,
                             int m, float* part, unsigned* arrivals, void* act, int cus, hipStream_t stream) {
  const CodesPlan p = plan_gemm_codes(m);
  // (act: bf16 activations [m rounded up to 128][k] then (X, -128 X) [same rows][k / G], for m > 64)
  uint16_t* xc = static_cast<uint16_t*>(act);
  float2* xt = reinterpret_cast<float2*>(static_cast<uint8_t*>(act) + gemm_codes_act_table(L, m));
#define UQ_CODES_CASE(SC, GR) \
  case SC * 1000 + GR:        \
    return launch_codes_m<SC, GR>(p, L, codes, params, x, y, m, part, arrivals, xc, xt, cus, stream);
  switch (L->scheme * 1000 + L->group) {
    UQ_CODES_CASE(UQ_INT2, 64)
    UQ_CODES_CASE(UQ_INT2, 128)
    UQ_CODES_CASE(UQ_INT4, 64)
    UQ_CODES_CASE(UQ_INT4, 128)
    UQ_CODES_CASE(UQ_INT8, 64)
    UQ_CODES_CASE(UQ_INT8, 128)
    default: return hipErrorInvalidValue;
  }
#undef UQ_CODES_CASE
}

}  // namespace uq
