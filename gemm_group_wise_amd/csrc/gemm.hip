// Fused group-wise dequant + GEMM on the bf16 matrix cores, for batched
// decode and prefill ("Ultra LLM Engine", Core Components > Fused Kernels:
// dequantized-weight GEMM during batched decode).
//
// y[m][n] = sum_k bf16(x[m][k]) * bf16(w'[n][k]), fp32 accumulation, where
// w' = fma(q, s, z) (INT-N) or C[q] * a (NF4) is the exact fp32 dequant and
// both casts round to nearest even.
//
// Two launches on the caller's stream:
//   1. x (fp16) -> bf16 into an activation workspace, once per call, so the
//      conversion is not repeated by every column tile.
//   2. The GEMM.  A workgroup is 8 waves (two per SIMD, so one wave's
//      dequant VALU work and LDS reads run under the other's MFMAs; on gfx950
//      a single wave does not overlap them well).  The workgroup owns BM rows
//      of x by BN = 64 * WGN weight rows; wave (wn, wk) owns weight rows
//      [64 wn, 64 wn + 64) of the tile and the KW-wide K slice wk of every
//      K step of KW * WGK.  Each wave keeps a BM x 64 fp32 accumulator
//      (v_mfma_f32_32x32x16_bf16 tiles) and the K slices are summed through
//      LDS at the end, so no partial sums go to memory.
//   * Activations: the bf16 tile of a K step (BM x KW*WGK) is copied
//     HBM -> LDS by global_load_lds_dwordx4 (no VGPR staging) into a ring of
//     kNB buffers (two by default: one step ahead), XOR-swizzled on 16-byte
//     chunks so the MFMA fragment reads are free of bank conflicts.
//   * Weights never pass through LDS: each lane loads the codes of its weight
//     row and K slice one step ahead into a ring of registers and dequantizes
//     them straight into MFMA B registers, 8 codes per MFMA, exactly once per
//     M tile.
//   * The cost of the loads goes by the number of cache lines they touch
//     more than by their bytes, and a burst of them stalls the issuing waves:
//     a step's loads go out in shares, one per MFMA sub-step of the step
//     before, and where one group covers the wave's whole K slice the group
//     parameters of both weight tiles come in one load.
//
// Lane layout of one wave's K slice of KW: lane l works on row (l % 32) of
// each 32-row tile and on codes [KW/2 * kh, KW/2 * (kh + 1)) with kh = l / 32;
// MFMA sub-step s (0 .. KW/16 - 1) takes codes 8s..8s+7 of that half on both
// the A and the B side (any consistent assignment of k within an MFMA gives
// the same dot product).
#include <mutex>
#include <vector>

#include "device_common.hpp"

namespace uq {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;
constexpr int kWaves = 8;
#ifndef UQ_GEMM_NB
#define UQ_GEMM_NB 2
#endif
constexpr int kNB = UQ_GEMM_NB;  // activation buffers = code register sets = prefetch distance + 1
static_assert(kNB == 2 || kNB == 4, "ring of two or four");

template <int BM, int WGN>
struct Tile {
  static constexpr int WGK = kWaves / WGN;              // K slices per step
  static constexpr int KW = (kNB == 2 || BM == 32) ? 64 : 32;  // k per wave per step
  static constexpr int SUB = KW / 16;                   // MFMA sub-steps per step
  static_assert(SUB >= 2, "the two weight tiles' loads go out in separate sub-steps");
  static constexpr int KS = KW * WGK;                   // k per step
  static constexpr int BN = 64 * WGN;                   // weight rows per workgroup
  static constexpr int TM = BM / 32;                    // 32-row MFMA tiles of x
  static constexpr int CPR = KS / 8;                    // 16-byte chunks per activation row
  static constexpr int BYTES = BM * KS * 2;             // one activation buffer
  static constexpr int LOADS = BYTES / (kThreads * 16); // 16-byte copies per thread per step
  static constexpr int RPI = kThreads / CPR;            // activation rows per copy round
  static_assert(kNB * BYTES <= 131072, "activation ring fits in LDS");
  static_assert(RPI % 8 == 0, "swizzle period");
  static_assert((WGK / 2) * WGN * TM * 2 * 16 * 64 * 4 <= kNB * BYTES, "K-slice reduction fits in LDS");
};

// The KW/2 codes of one lane for one weight row and K slice.
template <int S, int KW>
struct Codes {
  static constexpr int BYTES = KW / 2 * Fmt<S>::bits / 8;  // 4 .. 32
  static constexpr int W = BYTES / 4;
  uint32_t d[W];
};

// One load instruction per 16 bytes (or fewer): the count is part of the
// wait-count arithmetic in the kernel.
template <int S, int KW>
__device__ __forceinline__ void load_codes(Codes<S, KW>& c, const uint8_t* __restrict__ p) {
  constexpr int B = Codes<S, KW>::BYTES;
  if constexpr (B == 4) {
    c.d[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (B == 8) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    c.d[0] = v.x;
    c.d[1] = v.y;
  } else {
#pragma unroll
    for (int h = 0; h < B / 16; ++h) {
      const uint4 v = *reinterpret_cast<const uint4*>(p + 16 * h);
      c.d[4 * h] = v.x;
      c.d[4 * h + 1] = v.y;
      c.d[4 * h + 2] = v.z;
      c.d[4 * h + 3] = v.w;
    }
  }
}
template <int S, int KW>
constexpr int code_loads() {
  return Codes<S, KW>::BYTES <= 16 ? 1 : Codes<S, KW>::BYTES / 16;
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

// Group parameters of a lane's K slice, as fp32: (s, z), or (a, 0) for NF4.
// The lane's KW/2 codes span NGRP groups (two only for INT2 G16 with KW 64).
template <int S, int G, int KW>
struct Params {
  static constexpr int NGRP = G < KW / 2 ? KW / 2 / G : 1;
  float s[NGRP], z[NGRP];
};

// Codes 8s..8s+7 of the lane's KW/2 -> bf16(w') as an MFMA operand.
template <int S, int G, int KW>
__device__ __forceinline__ bf16x8 dequant8(const Codes<S, KW>& c, const Params<S, G, KW>& p, int s,
                                           const float* nf4) {
  constexpr int bits = Fmt<S>::bits;
  const int grp = G < KW / 2 ? (8 * s) / G : 0;
  const float sc = p.s[grp], zc = p.z[grp];
  float w[8];
  if constexpr (bits == 8) {
    const uint32_t d0 = c.d[2 * s], d1 = c.d[2 * s + 1];
    w[0] = __builtin_fmaf(ubyte_f32<0>(d0), sc, zc);
    w[1] = __builtin_fmaf(ubyte_f32<1>(d0), sc, zc);
    w[2] = __builtin_fmaf(ubyte_f32<2>(d0), sc, zc);
    w[3] = __builtin_fmaf(ubyte_f32<3>(d0), sc, zc);
    w[4] = __builtin_fmaf(ubyte_f32<0>(d1), sc, zc);
    w[5] = __builtin_fmaf(ubyte_f32<1>(d1), sc, zc);
    w[6] = __builtin_fmaf(ubyte_f32<2>(d1), sc, zc);
    w[7] = __builtin_fmaf(ubyte_f32<3>(d1), sc, zc);
  } else if constexpr (bits == 4) {
    const uint32_t d = c.d[s];
    const uint32_t lo = d & 0x0F0F0F0Fu, hi = (d >> 4) & 0x0F0F0F0Fu;  // codes 0,2,4,6 | 1,3,5,7
    if constexpr (S == UQ_NF4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[2 * i] = nf4[(lo >> (8 * i)) & 0xFu] * sc;
        w[2 * i + 1] = nf4[(hi >> (8 * i)) & 0xFu] * sc;
      }
    } else {
      w[0] = __builtin_fmaf(ubyte_f32<0>(lo), sc, zc);
      w[1] = __builtin_fmaf(ubyte_f32<0>(hi), sc, zc);
      w[2] = __builtin_fmaf(ubyte_f32<1>(lo), sc, zc);
      w[3] = __builtin_fmaf(ubyte_f32<1>(hi), sc, zc);
      w[4] = __builtin_fmaf(ubyte_f32<2>(lo), sc, zc);
      w[5] = __builtin_fmaf(ubyte_f32<2>(hi), sc, zc);
      w[6] = __builtin_fmaf(ubyte_f32<3>(lo), sc, zc);
      w[7] = __builtin_fmaf(ubyte_f32<3>(hi), sc, zc);
    }
  } else {  // 2 bits: codes 8s..8s+7 are 16 bits of one dword
    const uint32_t d = c.d[s >> 1] >> (16 * (s & 1));
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = __builtin_fmaf(float((d >> (2 * i)) & 3u), sc, zc);
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

template <int S, int G, int BM, int WGN>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ params,
                                                        const uint16_t* __restrict__ xb,
                                                        float* __restrict__ y, int n, int k, int m,
                                                        int tiles_m, int nblocks) {
  using T = Tile<BM, WGN>;
  constexpr int KW = T::KW;
  constexpr int bits = Fmt<S>::bits;
  constexpr int PB = param_bytes_per_group(S);
  constexpr int NGRP = Params<S, G, KW>::NGRP;
  // The activation buffers are separate LDS objects, so the compiler can tell
  // the copies into one from the fragment reads of another.
  constexpr int B23 = kNB == 4 ? T::BYTES : 16;
  __shared__ __attribute__((aligned(16))) uint8_t lds0[T::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[T::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds2[B23];
  __shared__ __attribute__((aligned(16))) uint8_t lds3[B23];
  __shared__ float nf4[16];
  auto buffer = [&](int i) __attribute__((always_inline)) {
    return i == 0 ? lds0 : i == 1 ? lds1 : i == 2 ? lds2 : lds3;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % WGN, wk = wave / WGN;
  const int b = xcd_order(blockIdx.x, nblocks);
  const int tile_m = b % tiles_m, tile_n = b / tiles_m;
  const int bm = tile_m * BM;
  const int steps = (k + T::KS - 1) / T::KS;
  const size_t rowb = size_t(k) * bits / 8;
  const int ng = k / G;
  if constexpr (S == UQ_NF4) {
    if (tid < 16) nf4[tid] = nf4_value(tid);
  }

  // Activation copy: thread tid moves 16-byte slot q = i * 512 + tid of the
  // step's tile (row q / CPR, physical chunk q % CPR, which holds logical
  // chunk (q % CPR) ^ (row & 7)).  RPI is a multiple of 8, so the logical
  // chunk is the same for every i.
  const int r0 = tid / T::CPR;
  const int cl = (tid % T::CPR) ^ (r0 & 7);
  const uint16_t* arow[T::LOADS];
#pragma unroll
  for (int i = 0; i < T::LOADS; ++i) {
    int r = bm + i * T::RPI + r0;
    r = r < m ? r : m - 1;  // rows past M: any valid row (their outputs are not stored)
    arow[i] = xb + size_t(r) * size_t(k);
  }

  // Weight rows of the lane's two 32-row tiles.
  const int kh = lane >> 5, r32 = lane & 31;
  const uint8_t* crow[2];
  const uint8_t* prow[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    int row = tile_n * T::BN + wn * 64 + t * 32 + r32;
    row = row < n ? row : n - 1;  // rows past N: computed, not stored
    crow[t] = codes + size_t(row) * rowb;
    prow[t] = params + size_t(row) * size_t(ng) * PB;
  }
  // When a group spans the wave's whole K slice (G >= KW), both halves of the
  // wave need the same group of both tiles' rows: one load fetches it (lanes
  // of half h take tile h) and a swap of the halves gives every lane both.
  constexpr bool kOneParamLoad = G >= KW;
  const uint8_t* prow_h = kh ? prow[1] : prow[0];

  f32x16 acc[T::TM][2];
#pragma unroll
  for (int a = 0; a < T::TM; ++a)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[a][t][j] = 0.0f;

  // Prefetch: step st's activation tile goes to buffer st % kNB and its codes
  // to register set st % kNB, issued kNB - 1 steps ahead (the step loop is
  // unrolled by kNB, so nothing is copied).  Each step issues the tile's
  // copies and then the codes, always (clamped to valid addresses past the
  // last step: loads under a branch make the compiler wait for every load
  // where the paths join).  Waiting for step st then means waiting until at
  // most the kNB - 2 later steps' loads are outstanding.
  constexpr int NT = T::LOADS;                         // copies per step
  constexpr int NC = 2 * code_loads<S, KW>() + (kOneParamLoad ? 1 : 2);  // code + parameter loads per step
  constexpr int NWAIT = (kNB - 2) * (NT + NC);
  static_assert(NWAIT < 64, "vmcnt field");
  Codes<S, KW> cs[kNB][2];        // [set][tile]
  uint32_t ps[kNB][2][NGRP];      // [set][tile][group]
  bool live[kNB] = {};

  // The loads of step st into set `set`, in SUB shares: share `part` holds the
  // tile copies i with i % SUB == part and, for part < 2, the codes (and
  // parameters) of weight tile `part`.  The shares are issued one per MFMA
  // sub-step, so the loads of a step reach the memory pipeline spread over the
  // previous step instead of in one burst after its barrier.
  auto issue = [&](int st, int set, int part) __attribute__((always_inline)) {
    int col = st * T::KS + 8 * cl;
    col = col < k ? col : 0;  // past K: any valid chunk (the weights there are zeroed)
    uint8_t* dst = buffer(set) + wave * 1024;
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i)
      if (i % T::SUB == part)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(arow[i] + col),
                                         (__attribute__((address_space(3))) void*)(dst + i * kThreads * 16), 16, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    const int kb = st * T::KS + KW * wk;  // the wave's K slice
    const int k0 = kb + KW / 2 * kh;      // the lane's half of it
    if (part == 0) live[set] = k0 < k;
    const int kc = k0 < k ? k0 : 0;       // past K: any valid slice (its weights are zeroed)
    static_assert(NGRP <= 2 && (NGRP == 1 || PB == 4), "parameter load");
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (t != part) continue;
      load_codes<S, KW>(cs[set][t], crow[t] + size_t(kc) * bits / 8);
      if constexpr (kOneParamLoad) {
        if (t == 0) {
          const int kq = kb < k ? kb : 0;
          const uint8_t* pp = prow_h + size_t(kq / G) * PB;
          if constexpr (PB == 4) ps[set][0][0] = *reinterpret_cast<const uint32_t*>(pp);
          else ps[set][0][0] = *reinterpret_cast<const uint16_t*>(pp);
        }
      } else {
        const uint8_t* pp = prow[t] + size_t(kc / G) * PB;
        if constexpr (NGRP == 2) {
          const uint2 v = *reinterpret_cast<const uint2*>(pp);  // kc / G is even: 8-byte aligned
          ps[set][t][0] = v.x;
          ps[set][t][1] = v.y;
        } else if constexpr (PB == 4) {
          ps[set][t][0] = *reinterpret_cast<const uint32_t*>(pp);
        } else {
          ps[set][t][0] = *reinterpret_cast<const uint16_t*>(pp);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // One K step from buffer and register set `set` = st % kNB.  Sub-steps are
  // software-pipelined: while sub-step s's MFMAs run, the wave reads sub-step
  // s+1's activation fragments and dequantizes its weights; the scheduling
  // hints interleave each MFMA with a share of that VALU work.
  auto step = [&](int st, int set) __attribute__((always_inline)) {
    // A plain s_barrier, not __syncthreads(): the fences of the latter wait for
    // every outstanding load (vmcnt(0)), the prefetched steps included.  The
    // waits go through the builtin so that the compiler's wait-count tracking
    // sees them (it then knows the tile's copies are done and adds no wait of
    // its own before the fragment reads).  The ds_reads of the previous step
    // have all been consumed by its MFMAs, so lgkmcnt(0) is immediate.
    __builtin_amdgcn_s_waitcnt(0x0F70 | (NWAIT & 15) | ((NWAIT >> 4) << 14));  // vmcnt(NWAIT), gfx9 encoding
    __builtin_amdgcn_s_waitcnt(0xC07F);                                         // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();  // step st's tile is in LDS for every wave; buffer (st-1) % kNB is free
    asm volatile("" ::: "memory");
    uint32_t praw[2][NGRP];
    if constexpr (kOneParamLoad) {
      const auto sw = __builtin_amdgcn_permlane32_swap(ps[set][0][0], ps[set][0][0], false, false);
      praw[0][0] = sw[0];  // tile 0's row (loaded by the lower half)
      praw[1][0] = sw[1];  // tile 1's row (loaded by the upper half)
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < NGRP; ++j) praw[t][j] = ps[set][t][j];
    }
    Params<S, G, KW> pc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < NGRP; ++j) {
        const uint32_t v = live[set] ? praw[t][j] : 0u;  // K slice past K: w' = 0
        if constexpr (S == UQ_NF4) {
          pc[t].s[j] = h2f(uint16_t(v));
          pc[t].z[j] = 0.0f;
        } else {
          pc[t].s[j] = h2f(uint16_t(v & 0xFFFFu));
          pc[t].z[j] = h2f(uint16_t(v >> 16));
        }
      }
    const Codes<S, KW> cc[2] = {cs[set][0], cs[set][1]};

    const uint8_t* Ab = buffer(set) + r32 * T::CPR * 16;
    auto afrag = [&](int a, int s) __attribute__((always_inline)) {
      const int chunk = ((KW / 8) * wk + (KW / 16) * kh + s) ^ (r32 & 7);
      return *reinterpret_cast<const bf16x8*>(Ab + (a * 32 * T::CPR + chunk) * 16);
    };
    bf16x8 acur[T::TM], bcur[2];
#pragma unroll
    for (int a = 0; a < T::TM; ++a) acur[a] = afrag(a, 0);
#pragma unroll
    for (int t = 0; t < 2; ++t) bcur[t] = dequant8<S, G, KW>(cc[t], pc[t], 0, nf4);
#pragma unroll
    for (int s = 0; s < T::SUB; ++s) {
      issue(st + kNB - 1, (set + kNB - 1) % kNB, s);
      bf16x8 anxt[T::TM], bnxt[2];
      if (s + 1 < T::SUB) {
#pragma unroll
        for (int a = 0; a < T::TM; ++a) anxt[a] = afrag(a, s + 1);
#pragma unroll
        for (int t = 0; t < 2; ++t) bnxt[t] = dequant8<S, G, KW>(cc[t], pc[t], s + 1, nf4);
      }
#pragma unroll
      for (int a = 0; a < T::TM; ++a)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[a][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(acur[a], bcur[t], acc[a][t], 0, 0, 0);
      if (s + 1 < T::SUB) {
#pragma unroll
        for (int q = 0; q < 2 * T::TM; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 48 / (2 * T::TM), 0);     // a share of the VALU
          if (q < T::TM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // and an LDS read
        }
#pragma unroll
        for (int a = 0; a < T::TM; ++a) acur[a] = anxt[a];
#pragma unroll
        for (int t = 0; t < 2; ++t) bcur[t] = bnxt[t];
      }
    }
  };

#pragma unroll
  for (int j = 0; j < kNB - 1; ++j)
#pragma unroll
    for (int p = 0; p < T::SUB; ++p) issue(j, j, p);
  // Whole rounds of kNB steps; the steps past K multiply by w' = 0.
  for (int st = 0; st < steps; st += kNB) {
#pragma unroll
    for (int u = 0; u < kNB; ++u) step(st + u, u);
  }

  // Sum the K slices: a halving tree through LDS (float4 per lane and
  // element group, lane-major so the partner wave reads what it wrote).
  constexpr int E4 = T::TM * 2 * 4;  // float4 per lane
  constexpr int SB = E4 * 64 * 16;    // bytes of one wave's partial sums
  static_assert(T::BYTES % SB == 0, "partial sums do not straddle the buffers");
  auto slot = [&](int sl) __attribute__((always_inline)) {
    const int off = sl * SB;
    return reinterpret_cast<float4*>(buffer(off / T::BYTES) + off % T::BYTES) + lane;
  };
  __syncthreads();
#pragma unroll
  for (int half = T::WGK / 2; half >= 1; half /= 2) {
    if (wk >= half && wk < 2 * half) {
      float4* dst = slot((wk - half) * WGN + wn);
#pragma unroll
      for (int a = 0; a < T::TM; ++a)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int j4 = 0; j4 < 4; ++j4)
            dst[((a * 2 + t) * 4 + j4) * 64] = make_float4(acc[a][t][4 * j4], acc[a][t][4 * j4 + 1],
                                                           acc[a][t][4 * j4 + 2], acc[a][t][4 * j4 + 3]);
    }
    __syncthreads();
    if (wk < half) {
      const float4* src = slot(wk * WGN + wn);
#pragma unroll
      for (int a = 0; a < T::TM; ++a)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int j4 = 0; j4 < 4; ++j4) {
            const float4 v = src[((a * 2 + t) * 4 + j4) * 64];
            acc[a][t][4 * j4] += v.x;
            acc[a][t][4 * j4 + 1] += v.y;
            acc[a][t][4 * j4 + 2] += v.z;
            acc[a][t][4 * j4 + 3] += v.w;
          }
    }
    __syncthreads();
  }
  if (wk != 0) return;

  // D layout of a 32x32 tile: lane l, element j -> row 8*(j/4) + 4*(l/32) + j%4
  // (an x row), column l % 32 (a weight row).
#pragma unroll
  for (int a = 0; a < T::TM; ++a)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int col = tile_n * T::BN + wn * 64 + t * 32 + r32;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int row = bm + a * 32 + 8 * (j / 4) + 4 * kh + (j % 4);
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

// Activation workspace, one per (device, stream) so calls on different
// streams never share it; calls on one stream are ordered by the stream.  A
// buffer that is outgrown stays allocated (a captured graph may still name
// it) until the process ends; growth is at least 2x, so the retired buffers
// add up to less than the live one.
struct Workspace {
  int device;
  hipStream_t stream;
  void* ptr;
  size_t bytes;
};
std::mutex g_ws_mutex;
std::vector<Workspace> g_ws;
std::vector<void*> g_ws_retired;

hipError_t activation_workspace(hipStream_t stream, size_t bytes, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  Workspace* w = nullptr;
  for (auto& it : g_ws)
    if (it.device == dev && it.stream == stream) w = &it;
  if (w && w->bytes >= bytes) {
    *out = w->ptr;
    return hipSuccess;
  }
  // No allocation while the stream is being captured into a graph.
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(stream, &cap);
  if (e != hipSuccess) return e;
  if (cap != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
  size_t want = bytes < (size_t(1) << 20) ? (size_t(1) << 20) : bytes;
  if (w && want < 2 * w->bytes) want = 2 * w->bytes;
  void* p = nullptr;
  e = hipMalloc(&p, want);
  if (e != hipSuccess) return e;
  if (w) {
    g_ws_retired.push_back(w->ptr);
    w->ptr = p;
    w->bytes = want;
  } else {
    g_ws.push_back(Workspace{dev, stream, p, want});
  }
  *out = p;
  return hipSuccess;
}

template <int S, int G, int BM, int WGN>
hipError_t launch(const uq_layout* L, const void* codes, const void* params, const uint16_t* xb,
                  float* y, int m, hipStream_t stream) {
  using T = Tile<BM, WGN>;
  int n = int(L->n), k = int(L->k);
  int tiles_m = (m + BM - 1) / BM;
  const int64_t tiles_n = (int64_t(n) + T::BN - 1) / T::BN;
  const int64_t nb = int64_t(tiles_m) * tiles_n;
  if (nb > 0x7fffffff) return hipErrorInvalidValue;
  int nblocks = int(nb);
  const uint8_t* c8 = static_cast<const uint8_t*>(codes);
  const uint8_t* p8 = static_cast<const uint8_t*>(params);
  void* args[] = {&c8, &p8, (void*)&xb, &y, &n, &k, &m, &tiles_m, &nblocks};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_kernel<S, G, BM, WGN>), dim3(unsigned(nblocks)),
                         dim3(kThreads), args, 0, stream);
}

template <int S, int G>
hipError_t launch_tiles(const uq_layout* L, const void* codes, const void* params, const uint16_t* xb,
                        float* y, int m, hipStream_t stream) {
  if (m <= 32) return launch<S, G, 32, 1>(L, codes, params, xb, y, m, stream);
  if (m <= 64) return launch<S, G, 64, 1>(L, codes, params, xb, y, m, stream);
  return launch<S, G, 128, 2>(L, codes, params, xb, y, m, stream);
}

}  // namespace

hipError_t launch_gemm(const uq_layout* L, const void* codes, const void* params, const uint16_t* x,
                       float* y, int m, hipStream_t stream) {
  const int64_t count = int64_t(m) * L->k;  // k % 32 == 0: whole 8-value pieces
  void* ws = nullptr;
  hipError_t e = activation_workspace(stream, size_t(count) * 2, &ws);
  if (e != hipSuccess) return e;
  uint16_t* xb = static_cast<uint16_t*>(ws);
  {
    int64_t count8 = count / 8;
    const int64_t want = (count8 + 255) / 256;
    const unsigned grid = unsigned(want < 1024 ? want : 1024);
    void* args[] = {(void*)&x, &xb, &count8};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&to_bf16_kernel), dim3(grid), dim3(256), args, 0, stream);
    if (e != hipSuccess) return e;
  }
  switch (L->scheme * 1000 + L->group) {
    case UQ_INT2 * 1000 + 16: return launch_tiles<UQ_INT2, 16>(L, codes, params, xb, y, m, stream);
    case UQ_INT2 * 1000 + 32: return launch_tiles<UQ_INT2, 32>(L, codes, params, xb, y, m, stream);
    case UQ_INT2 * 1000 + 64: return launch_tiles<UQ_INT2, 64>(L, codes, params, xb, y, m, stream);
    case UQ_INT2 * 1000 + 128: return launch_tiles<UQ_INT2, 128>(L, codes, params, xb, y, m, stream);
    case UQ_INT4 * 1000 + 32: return launch_tiles<UQ_INT4, 32>(L, codes, params, xb, y, m, stream);
    case UQ_INT4 * 1000 + 64: return launch_tiles<UQ_INT4, 64>(L, codes, params, xb, y, m, stream);
    case UQ_INT4 * 1000 + 128: return launch_tiles<UQ_INT4, 128>(L, codes, params, xb, y, m, stream);
    case UQ_INT8 * 1000 + 64: return launch_tiles<UQ_INT8, 64>(L, codes, params, xb, y, m, stream);
    case UQ_INT8 * 1000 + 128: return launch_tiles<UQ_INT8, 128>(L, codes, params, xb, y, m, stream);
    case UQ_NF4 * 1000 + 64: return launch_tiles<UQ_NF4, 64>(L, codes, params, xb, y, m, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace uq
