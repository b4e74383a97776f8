// Fused group-wise dequant + GEMM on the bf16 matrix cores, for batched
// decode and prefill ("Ultra LLM Engine", Core Components > Fused Kernels:
// dequantized-weight GEMM during batched decode).
//
// y[m][n] = sum_k bf16(x[m][k]) * bf16(w'[n][k]), fp32 accumulation, where
// w' = fma(q, s, z) (INT-N) or C[q] * a (NF4) is the exact fp32 dequant and
// both casts round to nearest even.
//
// One or two launches on the caller's stream:
//   1. From 65 activation rows (INT4 and NF4 always; INT8 and INT2 on
//      128-row tiles): x (fp16) -> bf16 into an activation
//      workspace, once per call, so the conversion is not repeated by every
//      column tile (there the GEMM is bound by VALU issue).  Up to 64 rows
//      the GEMM is bound by memory latency instead; it stages the caller's
//      fp16 x and rounds each fragment to bf16 as it reads it from LDS (the
//      same bits), which saves the extra launch (~4.7 us at M = 16).
//   2. The GEMM.  A workgroup is 8 waves (two per SIMD, so one wave's
//      dequant VALU work and LDS reads run under the other's MFMAs; on gfx950
//      a single wave does not overlap them well).  The workgroup owns BM rows
//      of x by BN = 64 * WGN weight rows; wave (wn, wk) owns weight rows
//      [64 wn, 64 wn + 64) of the tile and the 32-wide K slice wk of every
//      K step of 32 * WGK.  Each wave keeps a BM x 64 fp32 accumulator
//      (v_mfma_f32_32x32x16_bf16 tiles) and the K slices are summed through
//      LDS at the end, so no partial sums go to memory.
//   * Everything a step needs is copied into LDS by global_load_lds (no VGPR
//     staging): the activation tile (BM x KS, from L2) two steps ahead into
//     a ring of three buffers (one step ahead into two where three do not
//     fit); the packed codes of the BN weight rows for the step (from HBM, so
//     with a longer wait) three steps ahead into a ring of four; and a window
//     of 16 or more groups of parameters per weight row, at least three steps
//     ahead into the other half of a two-window buffer.  The vector memory
//     pipeline charges about a cycle per four adjacent lanes and cache line
//     touched, so every copy is
//     laid out for four or more adjacent lanes to read one line: a per-lane
//     load of each lane's own codes (32 rows per instruction) costs 3-4x as
//     much for the same bytes.  Each lane then reads its 16 codes and its
//     group's parameters back from LDS (swizzled layouts, few bank
//     conflicts) and dequantizes them straight into MFMA B registers, exactly
//     once per M tile.  The copies of a step go out in two shares, one per
//     MFMA sub-step of the step before, not in one burst after its barrier.
//
// Lane layout of one wave's K slice of 32: lane l works on row (l % 32) of
// each 32-row weight tile and on codes [16 kh, 16 kh + 16) with kh = l / 32;
// MFMA sub-step s (0, 1) takes codes 8s..8s+7 of that half on both the A and
// the B side (any consistent assignment of k within an MFMA gives the same
// dot product).
#include <atomic>
#include <mutex>

#include "device_common.hpp"

namespace uq {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kKW = 32;          // k per wave per step: 16 codes per lane, two MFMA sub-steps
constexpr int kSUB = kKW / 16;
constexpr int kDC = 3;           // codes are copied this many steps ahead (from HBM: long latency)
constexpr int kNC = kDC + 1;     // code buffers

// Groups per parameter window: at least 16, and enough that a window spans
// kDC or more steps (the next window is copied kDC steps before it is used,
// into the buffer of the window before the current one).
constexpr int param_window(int G, int KS) {
  int w = 16;
  while (w * G < kDC * KS) w *= 2;
  return w;
}

template <int BM, int WGN, int NW>
struct Tile {
  static constexpr int NT = 64 * NW;                    // threads per workgroup
  static constexpr int WGK = NW / WGN;                  // K slices per step
  static constexpr int KS = kKW * WGK;                  // k per step (256 or 128)
  static constexpr int BN = 64 * WGN;                   // weight rows per workgroup
  static constexpr int TM = BM / 32;                    // 32-row MFMA tiles of x
  static constexpr int CPR = KS / 8;                    // 16-byte chunks per activation row
  static constexpr int ABYTES = BM * KS * 2;            // one activation buffer
  static constexpr int ALOADS = ABYTES / (NT * 16);    // 16-byte copies per thread per step
  static constexpr int RPI = NT / CPR;                  // activation rows per copy round
  static_assert((ALOADS >= 1 && ALOADS % kSUB == 0) || ALOADS == 1, "copies split over the sub-steps");
  static_assert(RPI % 16 == 0 && CPR >= 16, "swizzle period");
};

// The weight codes of one step in LDS: BN rows of RB bytes, in 16-byte pieces;
// piece p of row r sits at position p ^ swz(r) so that the 16 rows read
// together by a half-wave land on different banks.  Copied with 16-byte lanes
// (INT4, INT8; rows are 16-byte aligned) or 4-byte lanes (INT2, whose rows are
// only 8-byte aligned), eight or more lanes per 128-byte line.
template <int S, int KS, int BN, int NW>
struct CodeTile {
  static constexpr int bits = Fmt<S>::bits;
  static constexpr int RB = KS * bits / 8;              // bytes of one weight row per step
  static constexpr int PPR = RB / 16;                   // 16-byte pieces per row
  static constexpr int BYTES = BN * RB;
  static constexpr int EL = bits == 2 ? 4 : 16;         // bytes per lane per copy
  static constexpr int PER_WAVE = BYTES / (EL * 64 * NW);  // copies per wave per step
  static constexpr int SWZ_DIV = 16 / PPR;
  static constexpr int LANE_BYTES = kKW / 2 * bits / 8;  // codes of one lane: 4, 8 or 16 bytes
  static_assert(PPR >= 2 && PPR <= 16 && PER_WAVE >= 1, "code tile shape");
  __device__ static int swz(int r) { return (r / SWZ_DIV) & (PPR - 1); }
};

// Workgroup barrier for LDS only: this wave's LDS accesses complete
// (lgkmcnt(0)), then s_barrier.  __syncthreads() also fences global memory,
// which on gfx9 means waiting for every outstanding vector-memory load,
// including loads meant to stay in flight.  The empty asm statements stop
// the compiler from moving LDS accesses across.
__device__ __forceinline__ void wait_lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), gfx9 encoding
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Byte I of a dword to fp32 in one instruction.  (Written as shift-and-mask,
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

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2 v = {__bf16(a), __bf16(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// The 16 codes of one lane (one weight row, one half of the wave's K slice).
template <int S>
struct Codes {
  static constexpr int W = kKW / 2 * Fmt<S>::bits / 8 / 4;  // 1, 2 or 4 dwords
  uint32_t d[W];
};

template <int S>
__device__ __forceinline__ Codes<S> lds_codes(const uint8_t* p) {
  Codes<S> c;
  if constexpr (Codes<S>::W == 1) {
    c.d[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (Codes<S>::W == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    c.d[0] = v.x;
    c.d[1] = v.y;
  } else {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    c.d[0] = v.x;
    c.d[1] = v.y;
    c.d[2] = v.z;
    c.d[3] = v.w;
  }
  return c;
}

// A code q masked in place in a 16-bit half, at bit b with b + bits <= 10,
// reads as the fp16 subnormal q 2^(b-24): exact, and exact again in fp32.
// With the group scale taken as s 2^(24-b) (a power-of-two multiple, exact
// in fp32) one fused multiply-add gives (q 2^(b-24)) (s 2^(24-b)) + z =
// q s + z rounded once -- fma(q, s, z) bit for bit -- and the compiler
// reads both the half and z straight from their registers (v_fma_mix_f32),
// so no conversion of the code is spent.
__device__ __forceinline__ float f16_lo(uint32_t v) { return float(__builtin_bit_cast(f16x2, v)[0]); }
__device__ __forceinline__ float f16_hi(uint32_t v) { return float(__builtin_bit_cast(f16x2, v)[1]); }

// Codes 8s..8s+7 of the lane's 16 -> bf16(w') as an MFMA operand, with the
// lane's group parameters (s, z) -- (a, 0) for NF4 -- in fp32.
template <int S>
__device__ __forceinline__ bf16x8 dequant8(const Codes<S>& c, float sc, float zc, int s, const float* nf4) {
  constexpr int bits = Fmt<S>::bits;
  constexpr float k24 = 16777216.0f, k22 = 4194304.0f, k20 = 1048576.0f, k18 = 262144.0f;
  float w[8];
  if constexpr (bits == 8) {
    // code 2i + h of a dword: byte h of half i
    const float s24 = sc * k24;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t d = c.d[2 * s + t];
      const uint32_t e = d & 0x00FF00FFu, o = (d >> 8) & 0x00FF00FFu;
      w[4 * t + 0] = __builtin_fmaf(f16_lo(e), s24, zc);
      w[4 * t + 1] = __builtin_fmaf(f16_lo(o), s24, zc);
      w[4 * t + 2] = __builtin_fmaf(f16_hi(e), s24, zc);
      w[4 * t + 3] = __builtin_fmaf(f16_hi(o), s24, zc);
    }
  } else if constexpr (bits == 4) {
    const uint32_t d = c.d[s];
    if constexpr (S == UQ_NF4) {
      const uint32_t lo = d & 0x0F0F0F0Fu, hi = (d >> 4) & 0x0F0F0F0Fu;  // codes 0,2,4,6 | 1,3,5,7
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[2 * i] = nf4[(lo >> (8 * i)) & 0xFu] * sc;
        w[2 * i + 1] = nf4[(hi >> (8 * i)) & 0xFu] * sc;
      }
    } else {
      // nibble j of the dword is code j: halves hold codes (0,4) (1,5) at
      // bits 0 and 4, and after a shift by 8 codes (2,6) (3,7)
      const float s24 = sc * k24, s20 = sc * k20;
      const uint32_t d8 = d >> 8;
      const uint32_t m0 = d & 0x000F000Fu, m1 = d & 0x00F000F0u, m2 = d8 & 0x000F000Fu, m3 = d8 & 0x00F000F0u;
      w[0] = __builtin_fmaf(f16_lo(m0), s24, zc);
      w[4] = __builtin_fmaf(f16_hi(m0), s24, zc);
      w[1] = __builtin_fmaf(f16_lo(m1), s20, zc);
      w[5] = __builtin_fmaf(f16_hi(m1), s20, zc);
      w[2] = __builtin_fmaf(f16_lo(m2), s24, zc);
      w[6] = __builtin_fmaf(f16_hi(m2), s24, zc);
      w[3] = __builtin_fmaf(f16_lo(m3), s20, zc);
      w[7] = __builtin_fmaf(f16_hi(m3), s20, zc);
    }
  } else {
    // 2 bits: codes 8s..8s+7 are bytes 2s, 2s+1 of the lane's dword; spread
    // them to the low bytes of the two halves, codes (j, 4+j) at bit 2j
    const uint32_t p = __builtin_amdgcn_perm(0u, c.d[0], s ? 0x0C030C02u : 0x0C010C00u);
    const float sj[4] = {sc * k24, sc * k22, sc * k20, sc * k18};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t mj = p & (0x00030003u << (2 * j));
      w[j] = __builtin_fmaf(f16_lo(mj), sj[j], zc);
      w[4 + j] = __builtin_fmaf(f16_hi(mj), sj[j], zc);
    }
  }
  const uint4 v = make_uint4(pack_bf16(w[0], w[1]), pack_bf16(w[2], w[3]), pack_bf16(w[4], w[5]),
                             pack_bf16(w[6], w[7]));
  return __builtin_bit_cast(bf16x8, v);
}

// Workgroup order: the dispatcher deals workgroups to the 8 XCDs in turn
// (workgroup b to XCD b % 8); renumber them so that each XCD gets a contiguous
// run of tiles, and the M tiles that share a weight tile share an L2.
__device__ __forceinline__ int xcd_order(int b, int nb) {
  const int q = nb >> 3, r = nb & 7, x = b & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}

template <int S, int G, int BM, int WGN, int NW, bool XF>
__global__ __launch_bounds__(64 * NW) void gemm_kernel(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ params,
                                                        const uint16_t* __restrict__ xb,
                                                        float* __restrict__ y, int n, int k, int m,
                                                        int tiles_m, int nblocks, int ksplit,
                                                        float* __restrict__ part,
                                                        unsigned* __restrict__ arrivals) {
  using T = Tile<BM, WGN, NW>;
  using C = CodeTile<S, T::KS, T::BN, NW>;
  constexpr int bits = Fmt<S>::bits;
  constexpr int PB = param_bytes_per_group(S);
  constexpr int WIN = param_window(G, T::KS);     // groups per parameter window
  constexpr int SPW = WIN * G / T::KS;            // steps per parameter window
  constexpr int PPW = T::BN * WIN / (64 * NW);    // parameter copies per wave per window
  constexpr int PBYTES = T::BN * WIN * 4;         // one window: a dword slot per group
  static_assert(SPW >= kDC && PPW >= 1, "parameter window shape");
  static_assert(G >= kKW / 2, "a lane's 16 codes lie in one group");
  // VALU instructions the scheduler places between consecutive MFMAs of a
  // sub-step, over the 2 * TM MFMAs: for 128-row tiles per scheme, as
  // measured at M = 256 (INT8 N = 4096 29.4 / 28.1 us per call with 48 / 32,
  // NF4 N = 14336 60.3 / 58.8 us with 48 / 72; INT4 N = 11008 46.4 us with
  // 48, 47.4-48.1 with 32, 72 or 96); 32 for row tiles of up to 64.
  constexpr int kShare = T::TM <= 2 ? 32 : S == UQ_INT8 ? 32 : S == UQ_NF4 ? 72 : 48;
  // Activation buffers: three when they fit next to the code ring (the tile
  // of step st + 2 is copied during step st), else two (st + 1).  Copies
  // complete in issue order, so the activation look-ahead also bounds how
  // long the codes copied before it may stay in flight.
  constexpr int LDS_FIXED = 2 * T::ABYTES + kNC * C::BYTES + 2 * PBYTES + 256;
  constexpr int AB = LDS_FIXED + T::ABYTES <= 160 * 1024 ? 3 : 2;
  constexpr int UNROLL = AB == 3 ? 12 : kNC;  // steps per round: buffer indices are constants
  // Every buffer the steps read while copies into another one are in flight
  // is its own LDS object (the activation and code buffers), and the step
  // loop is unrolled so each index is a constant: the compiler can then tell
  // the copies into one buffer from the reads of another and adds no waits
  // of its own.  The two parameter windows share one object: they are read
  // only at the start of a step, before the step issues any copy.
  __shared__ __attribute__((aligned(16))) uint8_t act0[T::ABYTES];
  __shared__ __attribute__((aligned(16))) uint8_t act1[T::ABYTES];
  __shared__ __attribute__((aligned(16))) uint8_t act2[AB == 3 ? T::ABYTES : 16];
  __shared__ __attribute__((aligned(16))) uint8_t cod0[C::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t cod1[C::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t cod2[C::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t cod3[C::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t par[2 * PBYTES];
  __shared__ float nf4[16];
  static_assert(kNC == 4 && UNROLL % kNC == 0 && UNROLL % AB == 0, "buffer indices repeat every round");
  auto abuf = [&](int i) __attribute__((always_inline)) { return i == 0 ? act0 : i == 1 ? act1 : act2; };
  auto cbuf = [&](int i) __attribute__((always_inline)) {
    return i == 0 ? cod0 : i == 1 ? cod1 : i == 2 ? cod2 : cod3;
  };
  auto pbuf = [&](int i) __attribute__((always_inline)) { return par + i * PBYTES; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % WGN, wk = wave / WGN;
  const int b = xcd_order(blockIdx.x, nblocks);
  const int split = b % ksplit, tile = b / ksplit;
  const int tile_m = tile % tiles_m, tile_n = tile / tiles_m;
  const int bm = tile_m * BM, bn = tile_n * T::BN;
  // This workgroup's share of the K steps: [st0, st1), balanced over ksplit.
  const int steps = (k + T::KS - 1) / T::KS;
  const int st0 = split * steps / ksplit, st1 = (split + 1) * steps / ksplit;
  const size_t rowb = size_t(k) * bits / 8;
  const int ng = k / G;
  if constexpr (S == UQ_NF4) {
    if (tid < 16) nf4[tid] = nf4_value(tid);
  }
  auto grow = [&](int r) __attribute__((always_inline)) {
    const int row = bn + r;
    return row < n ? row : n - 1;  // rows past N: computed, not stored
  };

  // Activation copy: thread tid moves 16-byte slot q = i * NT + tid of the
  // step's tile (row q / CPR, physical chunk q % CPR, which holds logical
  // chunk (q % CPR) ^ (row & 15)).  RPI is a multiple of 16, so the logical
  // chunk is the same for every i.
  const int r0 = tid / T::CPR;
  const int cl = (tid % T::CPR) ^ (r0 & 15);
  // Sources are a base common to the workgroup plus a 32-bit lane offset per
  // copy.  From the bf16 workspace (whole 128-row tiles) rows past M are read
  // without clamping; from the caller's fp16 x (XF) they are clamped to row
  // M - 1.  Either way their outputs are not stored.
  const uint16_t* abase = xb + size_t(bm) * size_t(k);
  uint32_t alane[T::ALOADS];
#pragma unroll
  for (int i = 0; i < T::ALOADS; ++i) {
    int r = i * T::RPI + r0;
    if constexpr (XF) r = bm + r < m ? r : m - 1 - bm;
    alane[i] = uint32_t(r) * uint32_t(k);
  }

  // Code copy j of this wave: lane slot q -> row r = piece / PPR, logical
  // piece p = (piece % PPR) ^ swz(r); 4-byte lanes take dword q % 4 of it.
  const uint8_t* cbase = codes + size_t(bn) * rowb;
  uint32_t crow[C::PER_WAVE], cbyte[C::PER_WAVE];
#pragma unroll
  for (int j = 0; j < C::PER_WAVE; ++j) {
    const int q = (wave * C::PER_WAVE + j) * 64 + lane;
    const int piece = C::EL == 16 ? q : q / 4;
    const int sub = C::EL == 16 ? 0 : q % 4;
    const int r = piece / C::PPR;
    const int p = (piece % C::PPR) ^ C::swz(r);
    cbyte[j] = uint32_t(p * 16 + sub * 4);
    crow[j] = uint32_t(grow(r) - bn) * uint32_t(rowb);
  }

  // Parameter copy j of this wave: dword slot q -> row r = q / WIN, slot
  // d' = q % WIN holding group d = d' ^ f(r) of the window, f(r) = (r / 4) % 16.
  const uint8_t* pbase = params + size_t(bn) * size_t(ng) * PB;
  uint32_t prowoff[PPW];
  int pgrp[PPW];
#pragma unroll
  for (int j = 0; j < PPW; ++j) {
    const int q = (wave * PPW + j) * 64 + lane;
    const int r = q / WIN;
    pgrp[j] = (q % WIN) ^ ((r >> 2) & 15);
    prowoff[j] = uint32_t(grow(r) - bn) * uint32_t(ng * PB);
  }

  // What this lane reads from LDS each step, for its two 32-row weight tiles.
  const int kh = lane >> 5, r32 = lane & 31;
  int coff[2], prow[2], pswz[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int r = wn * 64 + t * 32 + r32;
    const int bo = (kKW * wk + kKW / 2 * kh) * bits / 8;  // byte of the row's step segment
    coff[t] = (r * C::PPR + ((bo / 16) ^ C::swz(r))) * 16 + bo % 16;
    prow[t] = r * WIN;
    pswz[t] = (r >> 2) & 15;
  }

  f32x16 acc[T::TM][2];
#pragma unroll
  for (int a = 0; a < T::TM; ++a)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[a][t][j] = 0.0f;

  // Copies.  Per step, in this order: the parameter window that opens kDC
  // steps later (when one does), the next step's activation tile (in kSUB
  // shares, one per MFMA sub-step), and the codes of the step kDC ahead.
  // Waiting at a step for all but the last PER_WAVE copies then covers
  // everything the step reads.  Copies past K come from valid (clamped)
  // addresses and are multiplied by w' = 0.
  auto issue_params = [&](int win) __attribute__((always_inline)) {
    uint8_t* pdst = pbuf(win & 1) + wave * PPW * 256;
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
      int g = win * WIN + pgrp[j];
      g = g < ng ? g : ng - 1;  // past the row's groups: any valid one (not read)
      const auto src = (const __attribute__((address_space(1))) void*)(pbase + (prowoff[j] + uint32_t(g * PB)));
      const auto dst = (__attribute__((address_space(3))) void*)(pdst + j * 256);
      if constexpr (PB == 4) __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
      else __builtin_amdgcn_global_load_lds(src, dst, 2, 0, 0);  // lands zero-extended in a dword
    }
  };
  auto issue_act = [&](int st, int set, int part) __attribute__((always_inline)) {
    int col = st * T::KS + 8 * cl;
    col = col < k ? col : 0;
    uint8_t* adst = abuf(set) + wave * 1024;
#pragma unroll
    for (int i = 0; i < T::ALOADS; ++i)
      if (part < 0 || i % kSUB == part)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(abase + (alane[i] + uint32_t(col))),
                                         (__attribute__((address_space(3))) void*)(adst + i * T::NT * 16), 16, 0, 0);
  };
  auto issue_codes = [&](int st, int cset) __attribute__((always_inline)) {
    uint8_t* cdst = cbuf(cset) + wave * C::PER_WAVE * 64 * C::EL;
#pragma unroll
    for (int j = 0; j < C::PER_WAVE; ++j) {
      uint32_t off = uint32_t(st) * C::RB + cbyte[j];
      off = off < rowb ? off : 0u;  // past the row: any valid bytes (their weights are zeroed)
      const auto src = (const __attribute__((address_space(1))) void*)(cbase + (crow[j] + off));
      const auto dst = (__attribute__((address_space(3))) void*)(cdst + j * 64 * C::EL);
      if constexpr (C::EL == 16) __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
      else __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
    }
  };
  // Copies a wave may still have in flight when a step starts: those the
  // step before issued for later steps (its codes, and with three activation
  // buffers its activation tile too).  Everything older -- including what
  // this step reads -- has landed.
  constexpr int INFLIGHT = C::PER_WAVE + (AB == 3 ? T::ALOADS : 0);
  auto wait_step = [&]() __attribute__((always_inline)) {
    // A plain s_barrier, not __syncthreads() (whose fences wait for every
    // copy); the waits go through the builtin so that the compiler's
    // wait-count tracking sees them.  The scheduling barriers keep the
    // previous step's MFMAs from being moved after the wait.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F70 | INFLIGHT);     // vmcnt(INFLIGHT), gfx9 encoding
    __builtin_amdgcn_s_waitcnt(0xC07F);                // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  static_assert(INFLIGHT < 16, "vmcnt field");

  // The lane's codes and group parameters of step st, read from LDS (during
  // the step before, once everything step st reads has landed).
  auto read_step = [&](int st, int cset, Codes<S> (&cc)[2], uint32_t (&pr)[2]) __attribute__((always_inline)) {
    const int k0 = st * T::KS + kKW * wk + kKW / 2 * kh;
    const int win = st / SPW;
    const int gi = (k0 / G) - win * WIN;  // the lane's group within the window
    const uint32_t* pw = reinterpret_cast<const uint32_t*>(par) + (win & 1) * (PBYTES / 4);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      pr[t] = pw[prow[t] + (gi ^ pswz[t])];
      cc[t] = lds_codes<S>(cbuf(cset) + coff[t]);
    }
  };

  Codes<S> ccur[2];
  uint32_t pcur[2];

  // One K step from activation buffer u % AB and code buffer u % kNC.  Sub-
  // steps are software-pipelined: while sub-step s's MFMAs run, the wave
  // reads sub-step s+1's activation fragments and dequantizes its weights;
  // the scheduling hints interleave each MFMA with a share of that VALU work.
  auto step = [&](int st, int u) __attribute__((always_inline)) {
    wait_step();  // everything step st reads is in LDS; the buffers of step st - 1 are free
    // The next step's codes and parameters have landed too (copied kDC - 1 or
    // more steps ago); read them now, before this step issues copies of its
    // own, so that no copy in flight can be mistaken for a writer of them.
    Codes<S> cnext[2];
    uint32_t pnext[2];
    read_step(st + 1, (u + 1) % kNC, cnext, pnext);
    const bool live = st < st1 && st * T::KS + kKW * wk + kKW / 2 * kh < k;
    float sc[2], zc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t v = live ? pcur[t] : 0u;  // past K: w' = 0
      if constexpr (S == UQ_NF4) {
        sc[t] = h2f(uint16_t(v));
        zc[t] = 0.0f;
      } else {
        sc[t] = h2f(uint16_t(v & 0xFFFFu));
        zc[t] = h2f(uint16_t(v >> 16));
      }
    }
    const Codes<S> cc[2] = {ccur[0], ccur[1]};

    const uint8_t* Ab = abuf(u % AB) + r32 * T::CPR * 16;
    auto afrag = [&](int a, int s) __attribute__((always_inline)) {
      const int chunk = ((kKW / 8) * wk + (kKW / 16) * kh + s) ^ (r32 & 15);
      if constexpr (XF) {  // fp16 in LDS: round to bf16 here (exact fp32 widening, then RNE)
        const uint4 h = *reinterpret_cast<const uint4*>(Ab + (a * 32 * T::CPR + chunk) * 16);
        const uint4 v = make_uint4(pack_bf16(h2f(uint16_t(h.x)), h2f(uint16_t(h.x >> 16))),
                                   pack_bf16(h2f(uint16_t(h.y)), h2f(uint16_t(h.y >> 16))),
                                   pack_bf16(h2f(uint16_t(h.z)), h2f(uint16_t(h.z >> 16))),
                                   pack_bf16(h2f(uint16_t(h.w)), h2f(uint16_t(h.w >> 16))));
        return __builtin_bit_cast(bf16x8, v);
      } else {
        return *reinterpret_cast<const bf16x8*>(Ab + (a * 32 * T::CPR + chunk) * 16);
      }
    };
    bf16x8 acur[T::TM], bcur[2];
#pragma unroll
    for (int a = 0; a < T::TM; ++a) acur[a] = afrag(a, 0);
#pragma unroll
    for (int t = 0; t < 2; ++t) bcur[t] = dequant8<S>(cc[t], sc[t], zc[t], 0, nf4);
#pragma unroll
    for (int s = 0; s < kSUB; ++s) {
      if (s == 0) {
        if ((st + kDC) % SPW == 0) issue_params((st + kDC) / SPW);
        issue_act(st + AB - 1, (u + AB - 1) % AB, 0);
      } else {
        issue_act(st + AB - 1, (u + AB - 1) % AB, s);
        if (s == kSUB - 1) issue_codes(st + kDC, (u + kDC) % kNC);
      }
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 anxt[T::TM], bnxt[2];
      if (s + 1 < kSUB) {
#pragma unroll
        for (int a = 0; a < T::TM; ++a) anxt[a] = afrag(a, s + 1);
#pragma unroll
        for (int t = 0; t < 2; ++t) bnxt[t] = dequant8<S>(cc[t], sc[t], zc[t], s + 1, nf4);
      }
#pragma unroll
      for (int a = 0; a < T::TM; ++a)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[a][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(acur[a], bcur[t], acc[a][t], 0, 0, 0);
      if (s + 1 < kSUB) {
#pragma unroll
        for (int q = 0; q < 2 * T::TM; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, kShare / (2 * T::TM), 0);  // a share of the VALU
          if (q < T::TM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // and an LDS read
        }
#pragma unroll
        for (int a = 0; a < T::TM; ++a) acur[a] = anxt[a];
#pragma unroll
        for (int t = 0; t < 2; ++t) bcur[t] = bnxt[t];
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      ccur[t] = cnext[t];
      pcur[t] = pnext[t];
    }
  };

  // Prologue: the window of step st0 (and the next one when the steps would
  // issue it less than kDC steps after st0, i.e. before this range starts),
  // the codes of steps st0 .. st0 + kDC - 1 and the activation tiles of
  // steps st0 .. st0 + AB - 2, in the order the steps' waits expect (what
  // "the step before st0" would have issued last).  Buffers are indexed by
  // the step's place in the range: codes st0 + j in buffer j % kNC,
  // activations in buffer j % AB.
  issue_params(st0 / SPW);
  if ((st0 / SPW + 1) * SPW < st0 + kDC) issue_params(st0 / SPW + 1);
#pragma unroll
  for (int j = 0; j + 1 < kDC; ++j) issue_codes(st0 + j, j);
#pragma unroll
  for (int j = 0; j + 1 < AB; ++j) issue_act(st0 + j, j, -1);
  issue_codes(st0 + kDC - 1, kDC - 1);
  wait_step();
  read_step(st0, 0, ccur, pcur);
  // Rounds of UNROLL steps, left after the range's last step (copies it
  // issued for later steps are drained below).
  for (int st = st0;;) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      step(st, u);
      if (++st >= st1) goto steps_done;
    }
  }
steps_done:

  // Sum the K slices: a halving tree through LDS (float4 per lane and element
  // group, lane-major so the partner wave reads what it wrote), over FP of the
  // wave's 2 * TM accumulator tiles (tile f = 2 a + t) at a time so that the
  // partial sums fit the activation buffers.
  constexpr int FB = 4 * 64 * 16;  // bytes of one accumulator tile of one wave
  constexpr int FP_FIT = 2 * T::ABYTES / ((T::WGK / 2) * WGN * FB);
  constexpr int FP = FP_FIT >= 2 * T::TM ? 2 * T::TM : FP_FIT >= 4 ? 4 : FP_FIT >= 2 ? 2 : 1;
  static_assert(FP_FIT >= 1 && (2 * T::TM) % FP == 0, "reduction passes");
  constexpr int SB = FP * FB;  // bytes of one wave's partial sums per pass
  static_assert(T::ABYTES % SB == 0 && (T::WGK / 2) * WGN * SB <= 2 * T::ABYTES, "partial sums fit");
  auto slot = [&](int sl) __attribute__((always_inline)) {
    const int off = sl * SB;
    return reinterpret_cast<float4*>(abuf(off / T::ABYTES) + off % T::ABYTES) + lane;
  };
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the copies of the step past the end
  __syncthreads();
#pragma unroll
  for (int f0 = 0; f0 < 2 * T::TM; f0 += FP) {
#pragma unroll
    for (int half = T::WGK / 2; half >= 1; half /= 2) {
      if (wk >= half && wk < 2 * half) {
        float4* dst = slot((wk - half) * WGN + wn);
#pragma unroll
        for (int f = 0; f < FP; ++f)
#pragma unroll
          for (int j4 = 0; j4 < 4; ++j4) {
            const f32x16& v = acc[(f0 + f) / 2][(f0 + f) % 2];
            dst[(f * 4 + j4) * 64] = make_float4(v[4 * j4], v[4 * j4 + 1], v[4 * j4 + 2], v[4 * j4 + 3]);
          }
      }
      __syncthreads();
      if (wk < half) {
        const float4* src = slot(wk * WGN + wn);
#pragma unroll
        for (int f = 0; f < FP; ++f)
#pragma unroll
          for (int j4 = 0; j4 < 4; ++j4) {
            const float4 v = src[(f * 4 + j4) * 64];
            f32x16& d = acc[(f0 + f) / 2][(f0 + f) % 2];
            d[4 * j4] += v.x;
            d[4 * j4 + 1] += v.y;
            d[4 * j4 + 2] += v.z;
            d[4 * j4 + 3] += v.w;
          }
      }
      __syncthreads();
    }
  }

  // D layout of a 32x32 tile: lane l, element j -> row 8*(j/4) + 4*(l/32) + j%4
  // (an x row), column l % 32 (a weight row).
  auto out_row = [&](int a, int j) __attribute__((always_inline)) { return bm + a * 32 + 8 * (j / 4) + 4 * kh + (j % 4); };
  auto out_col = [&](int t) __attribute__((always_inline)) { return bn + wn * 64 + t * 32 + r32; };

  // (Split only for row tiles up to 64: the summing pass keeps kGemmMaxSplit
  // values of BM * BN / NT elements per thread in registers.)
  if constexpr (BM <= 64) if (ksplit > 1) {
    // K split over ksplit (<= kGemmMaxSplit) workgroups: each writes its partial
    // tile to part[split], and the last of the tile's workgroups to arrive
    // (counted with one device-scope atomic per tile) adds the ksplit partial
    // tiles in split order and stores y, so the sum does not depend on which
    // one arrives last.  Nothing waits on another workgroup.  Each XCD has
    // its own L2, so the partial tiles are written and read with agent-scope
    // atomic accesses (coherence bit set: stores write through the L2, loads
    // do not hit a non-coherent line) instead of fences: an agent-scope
    // release / acquire fence writes back / invalidates the whole L2, evicting
    // the activations every other workgroup on that XCD is streaming.  The
    // ordering that a release / acquire pair would give comes from
    // s_waitcnt vmcnt(0) (the stores are acknowledged at agent scope) and the
    // barrier before the counter increment, and on the reader from issuing
    // the loads only after the increment returned the final count.  The last
    // workgroup also returns the tile's counter to zero for the next call.
    const size_t rows = size_t(tiles_m) * BM;
    if (wk == 0) {
      float* dst = part + size_t(split) * rows * size_t(n);
#pragma unroll
      for (int a = 0; a < T::TM; ++a)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int col = out_col(t);
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (col < n)
              __hip_atomic_store(dst + size_t(out_row(a, j)) * size_t(n) + col, acc[a][t][j], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        }
    }
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
    // All threads of the last workgroup: thread tid takes elements
    // e = i * NT + tid of the BM x BN tile (consecutive threads, consecutive
    // columns), issues the loads of every partial tile at once and then adds
    // them in split order.
    constexpr int E = BM * T::BN / T::NT;
    float v[kGemmMaxSplit][E];
#pragma unroll
    for (int sp = 0; sp < kGemmMaxSplit; ++sp) {
      const int spc = sp < ksplit ? sp : ksplit - 1;  // past ksplit: a valid address, value unused
      const float* src = part + (size_t(spc) * rows + size_t(bm)) * size_t(n);
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const int e = i * T::NT + tid;
        const int col = min(bn + e % T::BN, n - 1);
        v[sp][i] = __hip_atomic_load(src + size_t(e / T::BN) * size_t(n) + col, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
      }
    }
#pragma unroll
    for (int i = 0; i < E; ++i) {
      float sum = v[0][i];
#pragma unroll
      for (int sp = 1; sp < kGemmMaxSplit; ++sp) sum = sp < ksplit ? sum + v[sp][i] : sum;
      const int e = i * T::NT + tid;
      const int row = bm + e / T::BN, col = bn + e % T::BN;
      if (row < m && col < n) y[size_t(row) * size_t(n) + col] = sum;
    }
    return;
  }

  if (wk != 0) return;
#pragma unroll
  for (int a = 0; a < T::TM; ++a)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int col = out_col(t);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int row = out_row(a, j);
        if (row < m && col < n) y[size_t(row) * size_t(n) + col] = acc[a][t][j];
      }
    }
}

// x (fp16) -> bf16, round to nearest even; 8 values per thread and pass.
__global__ __launch_bounds__(256) void to_bf16_kernel(const uint16_t* __restrict__ x,
                                                      uint16_t* __restrict__ xb, int64_t count8) {
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < count8; i += stride) {
    const uint4 h = reinterpret_cast<const uint4*>(x)[i];
    uint4 o;
    o.x = pack_bf16(h2f(uint16_t(h.x)), h2f(uint16_t(h.x >> 16)));
    o.y = pack_bf16(h2f(uint16_t(h.y)), h2f(uint16_t(h.y >> 16)));
    o.z = pack_bf16(h2f(uint16_t(h.z)), h2f(uint16_t(h.z >> 16)));
    o.w = pack_bf16(h2f(uint16_t(h.w)), h2f(uint16_t(h.w >> 16)));
    reinterpret_cast<uint4*>(xb)[i] = o;
  }
}

// Workgroups of this kernel one CU holds at once (cached per kernel).
template <int S, int G, int BM, int WGN, int NW, bool XF>
int resident_per_cu() {
  static std::atomic<int> cached{0};
  int v = cached.load(std::memory_order_relaxed);
  if (v > 0) return v;
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(&gemm_kernel<S, G, BM, WGN, NW, XF>),
                                                   64 * NW, 0) != hipSuccess || occ < 1)
    occ = 1;
  cached.store(occ, std::memory_order_relaxed);
  return occ;
}

int device_cus() {
  static std::atomic<int> cached{0};
  int v = cached.load(std::memory_order_relaxed);
  if (v > 0) return v;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  cached.store(cus, std::memory_order_relaxed);
  return cus;
}

// K split for a plan (reasons with plan_gemm in uq_internal.h): ksplit = the
// workgroups the chip holds at once (CUs x workgroups per CU, from the
// kernel's LDS and registers) over the tiles, at most kGemmMaxSplit.  Row
// tiles of up to 64 only, at least two K steps per workgroup.
template <int S, int G>
int plan_ksplit(const GemmPlan& p, int64_t m, int64_t n, int64_t k) {
  if (m > 64 || p.bm > 64) return 1;
  const int64_t tiles = ((m + p.bm - 1) / p.bm) * ((n + 64 * p.wgn - 1) / (64 * p.wgn));
  if (tiles > kGemmMaxSplitTiles) return 1;
  const int64_t ks_step = 32 * 8 / p.wgn;
  const int64_t steps = (k + ks_step - 1) / ks_step;
  const int per_cu = p.bm == 64 ? resident_per_cu<S, G, 64, 1, 8, true>() : resident_per_cu<S, G, 32, 1, 8, true>();
  int64_t ks = int64_t(device_cus()) * per_cu / tiles;
  if (ks > kGemmMaxSplit) ks = kGemmMaxSplit;
  if (ks > steps / 2) ks = steps / 2;
  return ks > 1 ? int(ks) : 1;
}

template <int S, int G, int BM, int WGN, int NW, bool XF>
hipError_t launch(const uq_layout* L, const void* codes, const void* params, const uint16_t* xb,
                  float* y, int m, int ksplit, float* part, unsigned* arrivals, hipStream_t stream) {
  using T = Tile<BM, WGN, NW>;
  int n = int(L->n), k = int(L->k);
  int tiles_m = (m + BM - 1) / BM;
  const int64_t tiles_n = (int64_t(n) + T::BN - 1) / T::BN;
  const int64_t nb = int64_t(tiles_m) * tiles_n * ksplit;
  if (nb > 0x7fffffff) return hipErrorInvalidValue;
  int nblocks = int(nb);
  const uint8_t* c8 = static_cast<const uint8_t*>(codes);
  const uint8_t* p8 = static_cast<const uint8_t*>(params);
  void* args[] = {&c8, &p8, (void*)&xb, &y, &n, &k, &m, &tiles_m, &nblocks, &ksplit, &part, &arrivals};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_kernel<S, G, BM, WGN, NW, XF>), dim3(unsigned(nblocks)),
                         dim3(T::NT), args, 0, stream);
}

// ---- Up to 32 activation rows: codes streamed straight into registers ----
//
// Up to 32 rows the GEMM is bound by memory traffic and by the dequantizing
// arithmetic, not by the matrix cores, so it is organised like the GEMV: a
// workgroup of four waves owns 64 weight rows (16 per wave) and a K range
// (the K split), which it walks in blocks of XB -- requesting the whole range
// at once when it is at most NB blocks, else keeping one block's loads in
// flight while the previous block is multiplied:
//   * the loads of a block are its activations and its rows' group
//     parameters (consecutive lanes, consecutive groups of a row), then its
//     codes, whole rows per load (the wave's 16 rows' blocks, 1 KB per load
//     instruction), moved through a per-wave LDS area into the MFMA layout:
//     lane l takes weight row l % 16 and, of the row's 16-byte pieces of the
//     block, the pieces 4 q + l / 16 -- within an MFMA any k order serves as
//     long as A and B agree, and the activations are staged in the same
//     order;
//   * once they land, the activations are staged in LDS (fp16 -> bf16, round
//     to nearest even) with the parameters, in one of NBUF buffers (with
//     one, a barrier first lets every wave finish reading the previous
//     block);
//   * after one barrier the block's v_mfma_f32_16x16x32_bf16 run, each B
//     operand dequantized from the lane's codes exactly as in the pipelined
//     kernel (bf16(fma(q, s, z))), so the products are the same.
template <int S, int G, int TM, int XB_>
struct SGeo {
  static constexpr int BM = 16 * TM, BN = 64, NT = 256;
  static constexpr int bits = Fmt<S>::bits;
  static constexpr int PB = param_bytes_per_group(S);
  static constexpr int XB = XB_;                // K per block
  static constexpr int Q = XB / 4;              // codes of one lane per block
  static constexpr int CP = 128 / bits;         // codes in a 16-byte piece
  static constexpr int NJ = Q / 8;              // MFMAs per block and row tile
  static constexpr int QW = Q * bits / 32;      // code dwords of a lane per block
  static constexpr int XPITCH = XB * 2 + 16;
  static constexpr int XI = BM * XB / 8;        // 8-activation pieces staged per block
  static constexpr int XPT = XI / NT;
  static constexpr int NGB = XB / G;            // groups per block
  static constexpr int PPB = BN * NGB;          // parameters per block
  static constexpr int PPT = (PPB + NT - 1) / NT;
  static constexpr int RB = XB * bits / 8;       // code bytes of a weight row per block
  static constexpr int LPR = RB / 16;           // lanes reading one row's block (16 bytes each)
  static constexpr int RPI = 64 / LPR;          // rows per wave load instruction
  static constexpr int CPITCH = RB + 16;        // LDS bytes per row in a wave's code area
  static_assert(XI % NT == 0 && QW % 4 == 0 && NJ % 2 == 0 && Q % 16 == 0, "block geometry");
  static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0 && QW / 4 * RPI == 16, "code loads: 16 rows per wave");
};

// One block's loads, in registers until staged.
template <class Ge>
struct StreamLoads {
  uint4 x[Ge::XPT];
  uint32_t p[Ge::PPT];
  uint32_t run[Ge::QW];
};

template <int S, int G, int TM, int XB, int NB, int NBUF>
__global__ __launch_bounds__(256) void gemm_stream_kernel(const uint8_t* __restrict__ codes,
                                                          const uint8_t* __restrict__ params,
                                                          const uint16_t* __restrict__ x, float* __restrict__ y,
                                                          int n, int k, int m, int tiles_m, int ksplit,
                                                          float* __restrict__ part, unsigned* __restrict__ arrivals) {
  using Ge = SGeo<S, G, TM, XB>;
  constexpr int bits = Ge::bits, BM = Ge::BM, BN = Ge::BN, NT = Ge::NT, NJ = Ge::NJ;
  constexpr int QW = Ge::QW, NGB = Ge::NGB;
  __shared__ __attribute__((aligned(16))) uint8_t xs[NBUF][BM * Ge::XPITCH];
  __shared__ __attribute__((aligned(16))) uint32_t ps[NBUF][Ge::PPT * NT];  // PPB used, the rest written blindly
  __shared__ __attribute__((aligned(16))) uint8_t cs[4][16 * Ge::CPITCH];     // each wave's codes, row-major
  __shared__ float nf4[16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x;
  const int split = b % ksplit, tile = b / ksplit;
  const int tile_m = tile % tiles_m, tile_n = tile / tiles_m;
  const int bm = tile_m * BM, bn = tile_n * BN;
  const int nblk = k / XB;  // whole blocks only (the launcher sends other K to the pipelined kernel)
  const int b0 = split * nblk / ksplit, b1 = (split + 1) * nblk / ksplit;
  const int rowb = k * bits / 8;
  const int ng = k / G;
  const int l16 = lane & 15, kb = lane >> 4;
  // Code loads read whole rows: load i of a lane covers row RPI i + lane / LPR
  // of the wave's 16, bytes 16 (lane % LPR) of the row's block (rows past N
  // re-read row N - 1: computed, not stored).
  const uint8_t* cptr[QW / 4];
#pragma unroll
  for (int i = 0; i < QW / 4; ++i) {
    int r = bn + 16 * wave + Ge::RPI * i + lane / Ge::LPR;
    r = r < n ? r : n - 1;
    cptr[i] = codes + size_t(r) * size_t(rowb) + 16 * (lane % Ge::LPR);
  }
  uint8_t* cw = cs[wave];
  if constexpr (S == UQ_NF4) {
    if (tid < 16) nf4[tid] = nf4_value(tid);
  }

  // issue a block's loads (activation rows past M and weight rows past N
  // clamped to the last: loaded, never stored)
  auto issue = [&](StreamLoads<Ge>& ld, int blk) {
    const int k0 = blk * XB;
#pragma unroll
    for (int i = 0; i < Ge::XPT; ++i) {
      const int it = i * NT + tid;
      const int row = it / (XB / 8), c = it % (XB / 8);
      int mr = bm + row;
      mr = mr < m ? mr : m - 1;
      ld.x[i] = *reinterpret_cast<const uint4*>(x + size_t(mr) * size_t(k) + k0 + 8 * c);
    }
#pragma unroll
    for (int i = 0; i < Ge::PPT; ++i) {
      int q = i * NT + tid;
      q = q < Ge::PPB ? q : Ge::PPB - 1;
      int pr = bn + q / NGB;
      pr = pr < n ? pr : n - 1;
      const uint8_t* src = params + (size_t(pr) * size_t(ng) + k0 / G + q % NGB) * Ge::PB;
      if constexpr (Ge::PB == 4) ld.p[i] = load_stream<uint32_t>(src);
      else ld.p[i] = load_stream<uint16_t>(src);
    }
#pragma unroll
    for (int i = 0; i < QW / 4; ++i) {
      const uint4 v = load_stream<uint4>(cptr[i] + size_t(k0) * bits / 8);
      ld.run[4 * i] = v.x;
      ld.run[4 * i + 1] = v.y;
      ld.run[4 * i + 2] = v.z;
      ld.run[4 * i + 3] = v.w;
    }
  };
  // Move a block's codes from the row-contiguous load layout into the MFMA
  // layout through the wave's LDS area: lane (row l16, k-block kb) takes the
  // row's 16-byte pieces 4 q + kb.  Only the wave touches its area, and a
  // wave's LDS accesses complete in issue order; the empty asm statements
  // keep the compiler from moving them across each other.
  auto transpose = [&](const StreamLoads<Ge>& ld, uint32_t (&run)[QW]) {
    asm volatile("" ::: "memory");  // the previous block's reads came first
#pragma unroll
    for (int i = 0; i < QW / 4; ++i)
      *reinterpret_cast<uint4*>(cw + (Ge::RPI * i + lane / Ge::LPR) * Ge::CPITCH + 16 * (lane % Ge::LPR)) =
          make_uint4(ld.run[4 * i], ld.run[4 * i + 1], ld.run[4 * i + 2], ld.run[4 * i + 3]);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int q = 0; q < QW / 4; ++q) {
      const uint4 v = *reinterpret_cast<const uint4*>(cw + l16 * Ge::CPITCH + 16 * (4 * q + kb));
      run[4 * q] = v.x;
      run[4 * q + 1] = v.y;
      run[4 * q + 2] = v.z;
      run[4 * q + 3] = v.w;
    }
  };

  f32x4 yacc[TM];
#pragma unroll
  for (int a = 0; a < TM; ++a) yacc[a] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // stage a block's activations and parameters in LDS buffer `buf`: 8
  // activations -> bf16 at slot 32 j + 8 kb of their row, where position p of
  // the block is in piece p / CP, read by k-block (p / CP) % 4 as its code
  // c = (p / CP / 4) CP + p % CP, of MFMA c / 8.  (A buffer is written two
  // blocks after it was last read, past a barrier that follows the reads.)
  auto stage = [&](const StreamLoads<Ge>& ld, int buf, bool live) {
    uint8_t* xb = xs[buf];
#pragma unroll
    for (int i = 0; i < Ge::XPT; ++i) {
      const int it = i * NT + tid;
      const int row = it / (XB / 8), c = it % (XB / 8);
      const int p = 8 * c, kbs = (p / Ge::CP) % 4, j = ((p / Ge::CP / 4) * Ge::CP + p % Ge::CP) / 8;
      const uint4 h = ld.x[i];
      const uint4 v = make_uint4(pack_bf16(h2f(uint16_t(h.x)), h2f(uint16_t(h.x >> 16))),
                                 pack_bf16(h2f(uint16_t(h.y)), h2f(uint16_t(h.y >> 16))),
                                 pack_bf16(h2f(uint16_t(h.z)), h2f(uint16_t(h.z >> 16))),
                                 pack_bf16(h2f(uint16_t(h.w)), h2f(uint16_t(h.w >> 16))));
      *reinterpret_cast<uint4*>(xb + row * Ge::XPITCH + (32 * j + 8 * kbs) * 2) = live ? v : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < Ge::PPT; ++i) ps[buf][i * NT + tid] = ld.p[i];
  };
  // a block's MFMAs from LDS buffer `buf`, two at a time (one Codes of 16
  // codes each pair)
  auto compute = [&](const uint32_t (&run)[QW], int buf) {
    const uint8_t* xb = xs[buf];
    const uint32_t* prw = ps[buf] + (16 * wave + l16) * NGB;
#pragma unroll
    for (int jp = 0; jp < NJ / 2; ++jp) {
      Codes<S> cc;
#pragma unroll
      for (int w = 0; w < Codes<S>::W; ++w) cc.d[w] = run[jp * Codes<S>::W + w];
      const uint32_t pw = prw[((4 * (16 * jp / Ge::CP) + kb) * Ge::CP + (16 * jp) % Ge::CP) / G];
      float sc, zc;
      if constexpr (S == UQ_NF4) {
        sc = h2f(uint16_t(pw));
        zc = 0.0f;
      } else {
        sc = h2f(uint16_t(pw & 0xFFFFu));
        zc = h2f(uint16_t(pw >> 16));
      }
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const bf16x8 bv = dequant8<S>(cc, sc, zc, sub, nf4);
        const int j = 2 * jp + sub;
#pragma unroll
        for (int a = 0; a < TM; ++a) {
          const bf16x8 av =
              *reinterpret_cast<const bf16x8*>(xb + (16 * a + l16) * Ge::XPITCH + (32 * j + 8 * kb) * 2);
          yacc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, yacc[a], 0, 0, 0);
        }
      }
    }
  };

  if constexpr (NB > 0) {
    // The whole K range (at most NB blocks; the launcher guarantees it) is
    // requested up front, block by block, and multiplied as it lands.
    // Slots past the range reload the last block and multiply it by zero
    // activations (adding exact zeros to sums that start at +0), so the code
    // has no branch: every load is issued before the first wait and each
    // wait is an exact count.
    const int nb = b1 - b0;
    StreamLoads<Ge> ld[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      issue(ld[bb], b0 + (bb < nb ? bb : nb - 1));
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      uint32_t run[QW];
      transpose(ld[bb], run);
      if (NBUF == 1 && bb > 0) wait_lds_barrier();  // the buffer's last reads are done
      stage(ld[bb], bb % NBUF, bb < nb);
      wait_lds_barrier();
      compute(run, bb % NBUF);
    }
  } else {
    // One block in flight while the previous one is multiplied.
    StreamLoads<Ge> ld;
    issue(ld, b0);
    for (int blk = b0; blk < b1; ++blk) {
      const int buf = (blk - b0) % NBUF;
      if (NBUF == 1 && blk > b0) wait_lds_barrier();  // the buffer's last reads are done
      stage(ld, buf, true);
      uint32_t run[QW];
      transpose(ld, run);
      if (blk + 1 < b1) issue(ld, blk + 1);
      wait_lds_barrier();
      compute(run, buf);
    }
  }

  // D layout: lane l, element i -> activation row 4 (l / 16) + i of tile a, weight row l % 16 of the wave.
  const int col = bn + 16 * wave + l16;
  if (ksplit > 1) {
    // K split: as in the pipelined kernel (partial tiles with agent-scope
    // atomic stores, one arrival counter per tile, the last workgroup adds
    // the partial tiles in split order and returns the counter to zero).
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

int device_cus();

template <int S, int G, int TM, int XB, int NB, int NBUF>
hipError_t launch_stream_t(const uq_layout* L, const void* codes, const void* params, const uint16_t* x, float* y,
                           int m, float* part, unsigned* arrivals, hipStream_t stream) {
  using Ge = SGeo<S, G, TM, XB>;
  int n = int(L->n), k = int(L->k);
  int tiles_m = (m + Ge::BM - 1) / Ge::BM;
  const int64_t tiles = int64_t(tiles_m) * ((int64_t(n) + Ge::BN - 1) / Ge::BN);
  // K split: the workgroups the chip holds at once over the tiles, at most
  // kGemmMaxSplit (the workspace holds that many partial tiles of 32 rows),
  // at least two blocks each where K has them.
  int ksplit = 1;
  if (tiles <= kGemmMaxSplitTiles) {
    static std::atomic<int> cached{0};
    int occ = cached.load(std::memory_order_relaxed);
    if (occ <= 0) {
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
              &occ, reinterpret_cast<const void*>(&gemm_stream_kernel<S, G, TM, XB, NB, NBUF>), Ge::NT, 0) != hipSuccess ||
          occ < 1)
        occ = 1;
      cached.store(occ, std::memory_order_relaxed);
    }
    int64_t ks = int64_t(device_cus()) * occ / tiles;
    if (ks > kGemmMaxSplit) ks = kGemmMaxSplit;
    if (ks > k / XB / (NB == 0 ? 2 : 1)) ks = k / XB / (NB == 0 ? 2 : 1);
    ksplit = ks > 1 ? int(ks) : 1;
  }
  if (NB > 0) {
    // every split holds at most NB blocks
    const int nblk = k / XB;
    while (ksplit < kGemmMaxSplit && (nblk + ksplit - 1) / ksplit > NB) ++ksplit;
    if ((nblk + ksplit - 1) / ksplit > NB || ksplit > nblk) return hipErrorInvalidValue;
  }
  const int64_t nb = tiles * ksplit;
  if (nb > 0x7fffffff) return hipErrorInvalidValue;
  const uint8_t* c8 = static_cast<const uint8_t*>(codes);
  const uint8_t* p8 = static_cast<const uint8_t*>(params);
  void* args[] = {&c8, &p8, (void*)&x, &y, &n, &k, &m, &tiles_m, &ksplit, &part, &arrivals};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_stream_kernel<S, G, TM, XB, NB, NBUF>), dim3(unsigned(nb)),
                         dim3(Ge::NT), args, 0, stream);
}

template <int S, int G>
hipError_t launch_plan(const GemmPlan& p, const uq_layout* L, const void* codes, const void* params,
                       const uint16_t* xb, float* y, int m, float* part, unsigned* arrivals, hipStream_t stream) {
  if (p.bm == 128) return launch<S, G, 128, 2, 8, false>(L, codes, params, xb, y, m, p.ksplit, part, arrivals, stream);
  if (p.bm == 64 && !p.xf) return launch<S, G, 64, 1, 8, false>(L, codes, params, xb, y, m, p.ksplit, part, arrivals, stream);
  if (p.bm == 64) return launch<S, G, 64, 1, 8, true>(L, codes, params, xb, y, m, p.ksplit, part, arrivals, stream);
  return launch<S, G, 32, 1, 8, true>(L, codes, params, xb, y, m, p.ksplit, part, arrivals, stream);
}

}  // namespace

// ---- Fixed scratch for uq_gemm_noalloc (callers that cannot allocate) ----
//
// One file-scope device array per GPU the library runs on, held until the
// process ends.  In host code the array's name is not a device address: its
// address on each device comes from hipGetSymbolAddress, taken once per
// device (with that device current) and kept; only that pointer is passed to
// kernels.  Every uq_gemm_noalloc call on a device shares the array, so such
// calls must not overlap on one device.
static __device__ __align__(256) uint8_t scratch[kGemmScratchBytes];

// Zero `words` 16-byte words at p (the arrival counters, once per device).
__global__ __launch_bounds__(256) void zero_kernel(uint4* __restrict__ p, int64_t words) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < words) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices];  // per device: the array's device address, once initialised
}  // namespace

hipError_t gemm_scratch(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    // The counters must start at zero (each call leaves them so); clear them
    // once, by a kernel on the call's stream, ahead of the first GEMM.
    int64_t words = int64_t(kGemmMaxSplitTiles) * 4 / 16;
    uint4* p = static_cast<uint4*>(ptr);
    void* args[] = {&p, &words};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&zero_kernel), dim3(unsigned((words + 255) / 256)), dim3(256),
                        args, 0, stream);
    if (e != hipSuccess) return e;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

hipError_t launch_gemm(const uq_layout* L, const void* codes, const void* params, const uint16_t* x,
                       float* y, int m, void* workspace, hipStream_t stream) {
  GemmPlan plan = plan_gemm(m, L->n, L->scheme);
#define UQ_GEMM_CASE(SC, GR) \
  case SC * 1000 + GR: plan.ksplit = plan_ksplit<SC, GR>(plan, m, L->n, L->k); break;
  switch (L->scheme * 1000 + L->group) {
    UQ_GEMM_CASE(UQ_INT2, 16)
    UQ_GEMM_CASE(UQ_INT2, 32)
    UQ_GEMM_CASE(UQ_INT2, 64)
    UQ_GEMM_CASE(UQ_INT2, 128)
    UQ_GEMM_CASE(UQ_INT4, 32)
    UQ_GEMM_CASE(UQ_INT4, 64)
    UQ_GEMM_CASE(UQ_INT4, 128)
    UQ_GEMM_CASE(UQ_INT8, 32)
    UQ_GEMM_CASE(UQ_INT8, 64)
    UQ_GEMM_CASE(UQ_INT8, 128)
    UQ_GEMM_CASE(UQ_NF4, 64)
    default: return hipErrorInvalidValue;
  }
#undef UQ_GEMM_CASE
  // The caller's workspace (validated to hold gemm_workspace(L, m).total
  // bytes): arrival counters, bf16 x in whole 128-row tiles unless the GEMM
  // reads the caller's fp16 x, and the partial tiles of a K split.  The GEMM
  // reads workspace rows past M without clamping (their products are never
  // stored).
  const GemmWorkspace wl = gemm_workspace(L, m);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  unsigned* arrivals = reinterpret_cast<unsigned*>(ws + wl.counters);
  uint16_t* xb = plan.xf ? const_cast<uint16_t*>(x) : reinterpret_cast<uint16_t*>(ws + wl.act);
  float* part = reinterpret_cast<float*>(ws + wl.part);
  if (m <= 32 && L->k % 256 == 0) {
    // K up to 4096 in blocks of 512: a workgroup requests its whole K range
    // (at most two blocks) at once; other K streams blocks of 256 with one
    // in flight.  (Measured on MI355X, INT4 G128 K4096 N11008 at 16 rows:
    // 14.4 us with four blocks of 256, 13.0 us with two of 512 in one LDS
    // buffer; at 32 rows 18.1 -> 16.3 us.)
    const bool all_in = L->k <= 4096 && L->k % 512 == 0;
#define UQ_STREAM_CASE(SC, GR)                                                                          \
  case SC * 1000 + GR:                                                                                  \
    if (all_in)                                                                                         \
      return m <= 16 ? launch_stream_t<SC, GR, 1, 512, 2, 1>(L, codes, params, x, y, m, part, arrivals, stream) \
                     : launch_stream_t<SC, GR, 2, 512, 2, 1>(L, codes, params, x, y, m, part, arrivals, stream); \
    return m <= 16 ? launch_stream_t<SC, GR, 1, 256, 0, 2>(L, codes, params, x, y, m, part, arrivals, stream)     \
                   : launch_stream_t<SC, GR, 2, 256, 0, 2>(L, codes, params, x, y, m, part, arrivals, stream);
    switch (L->scheme * 1000 + L->group) {
      UQ_STREAM_CASE(UQ_INT2, 16)
      UQ_STREAM_CASE(UQ_INT2, 32)
      UQ_STREAM_CASE(UQ_INT2, 64)
      UQ_STREAM_CASE(UQ_INT2, 128)
      UQ_STREAM_CASE(UQ_INT4, 32)
      UQ_STREAM_CASE(UQ_INT4, 64)
      UQ_STREAM_CASE(UQ_INT4, 128)
      UQ_STREAM_CASE(UQ_INT8, 32)
      UQ_STREAM_CASE(UQ_INT8, 64)
      UQ_STREAM_CASE(UQ_INT8, 128)
      UQ_STREAM_CASE(UQ_NF4, 64)
      default: return hipErrorInvalidValue;
    }
#undef UQ_STREAM_CASE
  }
  if (!plan.xf) {
    int64_t count8 = int64_t(m) * L->k / 8;  // k % 32 == 0: whole 8-value pieces
    const int64_t want = (count8 + 255) / 256;
    const unsigned grid = unsigned(want < 1024 ? want : 1024);
    void* args[] = {(void*)&x, &xb, &count8};
    const hipError_t e =
        hipLaunchKernel(reinterpret_cast<const void*>(&to_bf16_kernel), dim3(grid), dim3(256), args, 0, stream);
    if (e != hipSuccess) return e;
  }
#define UQ_GEMM_CASE(SC, GR) \
  case SC * 1000 + GR: return launch_plan<SC, GR>(plan, L, codes, params, xb, y, m, part, arrivals, stream);
  switch (L->scheme * 1000 + L->group) {
    UQ_GEMM_CASE(UQ_INT2, 16)
    UQ_GEMM_CASE(UQ_INT2, 32)
    UQ_GEMM_CASE(UQ_INT2, 64)
    UQ_GEMM_CASE(UQ_INT2, 128)
    UQ_GEMM_CASE(UQ_INT4, 32)
    UQ_GEMM_CASE(UQ_INT4, 64)
    UQ_GEMM_CASE(UQ_INT4, 128)
    UQ_GEMM_CASE(UQ_INT8, 32)
    UQ_GEMM_CASE(UQ_INT8, 64)
    UQ_GEMM_CASE(UQ_INT8, 128)
    UQ_GEMM_CASE(UQ_NF4, 64)
    default: return hipErrorInvalidValue;
  }
#undef UQ_GEMM_CASE
}

}  // namespace uq
