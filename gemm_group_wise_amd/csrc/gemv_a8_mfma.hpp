// Activation-quantized GEMV on the integer matrix cores, 2 to 8 activation
// rows of INT4 and INT8 weights with groups of 32, 64 or 128 and of INT2
// weights with groups of 16 ("Ultra LLM Engine", Core Components
// > Quantized Model: the quantized layers quantize their activations on the
// fly; Fused Kernels: the decode GEMV).
//
// The arithmetic is the dot-product A8 kernel's (reading R-AD): activations
// quantized to int8 per (activation row, weight group) exactly as there, and
//     y[m][n] = sum_g s_x * (s * D + z * Q),  D = sum q_w * q_x,  Q = sum q_x,
// with D and Q exact integers and only the per-group scaling in fp32.  Here
// D comes from v_mfma_i32_16x16x64_i8: one chain of G / 64 MFMAs per group,
// int32 accumulation (|D| < 2^22); 32-code groups take one
// v_mfma_i32_16x16x32_i8 each (8 codes per lane), and so do 16-code groups,
// two to a k range, each with the other group's B lanes zeroed.
//   * B operand: the codes as bytes, INT8 with the sign bit flipped (q - 128,
//     corrected by 128 * Q), INT4 nibbles spread to bytes with two masks;
//   * A operand: the activation codes, staged in LDS in the order the
//     unpacked weight bytes take (INT4: even codes, then odd codes, of each
//     8), with (s_x, Q) per (group, activation row);
//   * MFMA lane layout (16x16x64): lane l holds A[row l % 16][k-block l / 16]
//     and B[k-block l / 16][column l % 16], 16 consecutive k per lane (8 on the 16x16x32);
//     D rows 4 (l / 16) .. + 3 are activation rows, column l % 16 a weight row.
// Work split as in the fp16 matrix-core GEMV (gemv_mfma.hpp): a workgroup of
// W waves owns 16 weight rows, wave w takes the w-th of W equal slices of
// every row (whole 128-byte blocks; K padded with zero activations), codes
// and parameters are loaded densely and moved through a per-wave LDS block
// into the MFMA layout, the activations are quantized into LDS once per
// workgroup, and the W partial tiles are added in wave order at the end.
// The sums of a row do not depend on how many activation rows the call has:
// the rows of calls with 2 to 8 activation rows agree bit for bit.
#pragma once

#include <type_traits>

#include "device_common.hpp"

namespace uq {
namespace {

constexpr int kA8mBlock = 128;         // code bytes per row per block (two dense loads of 8 rows)
constexpr int kA8mRowPitch = 144;      // LDS bytes per row of a block: 16 rows of 16-byte reads, distinct banks
constexpr int kA8mXBytes = 64 * 1024;  // most LDS the staged activation codes may take

template <int S, int G>
constexpr bool a8_mfma_scheme() {
  return ((S == UQ_INT4 || S == UQ_INT8) && (G == 32 || G == 64 || G == 128)) || (S == UQ_INT2 && G == 16);
}

template <int S, int G, int MT, int W, int NBLK>
struct A8mGeo {
  static constexpr int bits = Fmt<S>::bits;
  static constexpr int KM = G <= 32 ? 32 : 64;               // k per MFMA (16x16x32 for 16- and 32-code groups)
  static constexpr int KL = KM / 4;                          // k per lane per MFMA
  static constexpr int QB = NBLK * kA8mBlock;                // code bytes per row per wave
  static constexpr int QK = QB * 8 / bits;                   // k per wave
  static constexpr int KP = W * QK;                          // padded K of a launch
  static constexpr int GPW = QK / G;                         // groups per wave
  static constexpr int NG = KP / G;                          // groups of the padded K
  static constexpr int MPB = kA8mBlock * 8 / bits / KM;      // k ranges of one MFMA per block
  // 16-code groups (INT2 G16) share a k range two to an MFMA: each group's
  // MFMA takes the range with the other group's half of the B lanes zeroed
  static constexpr bool HALF = G < KM;
  static constexpr int MPG = HALF ? 1 : G / KM;              // MFMAs per group
  static constexpr int GPB = HALF ? MPB * (KM / G) : MPB / MPG;  // groups per block
  static constexpr int QP = GPW * 4;                         // parameter bytes per row per wave
  static constexpr int PP = QP + 16;                         // their LDS pitch per row
  static constexpr int XPITCH = KP + 16;                     // LDS bytes per staged activation row
  static constexpr int X_BYTES = MT * XPITCH;
  static constexpr int T_BYTES = MT * NG * 8;                // (s_x, Q) per (group, row)
  static constexpr int B_BYTES = 16 * kA8mRowPitch;          // one wave's block
  static constexpr int P_BYTES = 16 * PP;                    // one wave's parameters
  static constexpr int LDS = X_BYTES + T_BYTES + W * (B_BYTES + P_BYTES);
  static constexpr int PLOADS = (16 * QP + 1023) / 1024;     // 16-byte parameter loads per lane
  static constexpr int XPIECES = MT * KP / 16;               // 16-activation pieces quantized
  static constexpr int PIECES = (XPIECES + 64 * W - 1) / (64 * W);  // per thread
  // An MFMA lies in one group and a wave holds whole groups; whole 16-byte
  // parameter slots per row; a group's pieces are consecutive lanes of one
  // wave; the staged codes fit their LDS budget.
  static constexpr bool ok = a8_mfma_scheme<S, G>() && (G % KM == 0 || KM == 2 * G) && QK % G == 0 && QP % 16 == 0 &&
                             64 % (G / 16) == 0 && X_BYTES <= kA8mXBytes && B_BYTES + P_BYTES >= 1024 &&
                             LDS <= 160 * 1024;
};

// Position p (0..15) of a 16-code piece in the order the unpacked B bytes
// take -> the code it holds.  INT4: a dword's low nibbles (codes 0, 2, 4, 6)
// then its high nibbles (1, 3, 5, 7), per 8 codes.
template <int S>
__device__ __forceinline__ constexpr int a8m_src(int p) {
  if constexpr (S == UQ_INT4) return (p & 8) + 2 * (p & 3) + ((p >> 2) & 1);
  else if constexpr (S == UQ_INT2) return (p & 8) + 4 * (p & 1) + ((p >> 1) & 3);  // per 8: 0 4 1 5 2 6 3 7
  else return p;
}

// Quantize one 16-value piece with its group's max |x| a, as quantize16 does
// (t = fp32(x * fp32(127 / a)), rint to even, clamped to +-127), in fewer
// instructions: t is clamped first (the same result: rint is monotonic and
// +-127 are integers), then 1.5 * 2^23 + t rounds t to an integer in the low
// mantissa bits (fp32 addition rounds to nearest even), whose low byte is the
// two's-complement code.  The bytes are gathered with v_perm_b32 in the B
// operand's order, and Q (the piece's code sum) comes from v_dot4 with ones.
template <int S>
__device__ __forceinline__ void quantize_piece(const float (&v)[16], float a, uint32_t (&packed)[4], int& qs) {
  const float r = a > 0.0f ? 127.0f / a : 0.0f;
  uint32_t u[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float t = __builtin_amdgcn_fmed3f(v[e] * r, -127.0f, 127.0f);
    u[e] = __float_as_uint(t + 12582912.0f);
  }
  qs = 0;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    // bytes 4d..4d+3 hold codes a8m_src(4d..4d+3): (b0 of u0, b0 of u1) then (b0 of u2, b0 of u3)
    const uint32_t lo = __builtin_amdgcn_perm(u[a8m_src<S>(4 * d + 1)], u[a8m_src<S>(4 * d)], 0x0C0C0400u);
    const uint32_t hi = __builtin_amdgcn_perm(u[a8m_src<S>(4 * d + 3)], u[a8m_src<S>(4 * d + 2)], 0x0C0C0400u);
    packed[d] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    qs = __builtin_amdgcn_sdot4(int(packed[d]), 0x01010101, qs, false);
  }
}

typedef int i32x4v __attribute__((ext_vector_type(4)));

// One group's chain of N MFMAs from zero, as one inline-asm statement with
// the accumulator tied to the destination and explicit wait states (the
// same discipline as the fp16 matrix-core GEMV, whose builtin code
// generation returned wrong lanes for some instantiations).
#define UQ_A8M_PRE "s_nop 7\n\ts_nop 7\n\t"
#define UQ_A8M_POST "\n\ts_nop 7\n\ts_nop 7\n\ts_nop 4"
template <int N>
__device__ __forceinline__ void a8_chain(i32x4v& acc, const uint4 (&a)[N], const uint4 (&b)[N]) {
  static_assert(N == 1 || N == 2, "chains of 1 or 2 MFMAs");
  i32x4v av[N], bv[N];
#pragma unroll
  for (int j = 0; j < N; ++j) {
    av[j] = __builtin_bit_cast(i32x4v, a[j]);
    bv[j] = __builtin_bit_cast(i32x4v, b[j]);
  }
  if constexpr (N == 1) {
    asm volatile(UQ_A8M_PRE "v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" UQ_A8M_POST : "+v"(acc) : "v"(av[0]), "v"(bv[0]));
  } else {
    asm volatile(UQ_A8M_PRE "v_mfma_i32_16x16x64_i8 %0, %1, %2, %0\n\t" UQ_A8M_PRE
                 "v_mfma_i32_16x16x64_i8 %0, %3, %4, %0" UQ_A8M_POST
                 : "+v"(acc) : "v"(av[0]), "v"(bv[0]), "v"(av[1]), "v"(bv[1]));
  }
}
// Several groups' chains in one statement with independent accumulators
// interleaved, so that the wait states are paid once for all of them (each
// dependent MFMA still follows the one it adds to by sixteen or more).
template <int C>
__device__ __forceinline__ void a8_chains1(i32x4v (&acc)[C], const uint4 (&a)[C], const uint4 (&b)[C]) {
  static_assert(C == 2 || C == 4, "two or four one-MFMA chains");
  i32x4v av[C], bv[C];
#pragma unroll
  for (int j = 0; j < C; ++j) {
    av[j] = __builtin_bit_cast(i32x4v, a[j]);
    bv[j] = __builtin_bit_cast(i32x4v, b[j]);
  }
  if constexpr (C == 2) {
    asm volatile(UQ_A8M_PRE "v_mfma_i32_16x16x64_i8 %0, %2, %3, %0\n\tv_mfma_i32_16x16x64_i8 %1, %4, %5, %1" UQ_A8M_POST
                 : "+v"(acc[0]), "+v"(acc[1]) : "v"(av[0]), "v"(bv[0]), "v"(av[1]), "v"(bv[1]));
  } else {
    asm volatile(UQ_A8M_PRE "v_mfma_i32_16x16x64_i8 %0, %4, %5, %0\n\tv_mfma_i32_16x16x64_i8 %1, %6, %7, %1\n\t"
                 "v_mfma_i32_16x16x64_i8 %2, %8, %9, %2\n\tv_mfma_i32_16x16x64_i8 %3, %10, %11, %3" UQ_A8M_POST
                 : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])
                 : "v"(av[0]), "v"(bv[0]), "v"(av[1]), "v"(bv[1]), "v"(av[2]), "v"(bv[2]), "v"(av[3]), "v"(bv[3]));
  }
}
// 32-code groups: one v_mfma_i32_16x16x32_i8 per group (8 codes per lane),
// up to four groups' MFMAs in one statement.
template <int C>
__device__ __forceinline__ void a8_chains32(i32x4v (&acc)[C], const uint2 (&a)[C], const uint2 (&b)[C]) {
  static_assert(C == 2 || C == 4, "two or four one-MFMA chains");
  long av[C], bv[C];
#pragma unroll
  for (int j = 0; j < C; ++j) {
    av[j] = __builtin_bit_cast(long, a[j]);
    bv[j] = __builtin_bit_cast(long, b[j]);
  }
  if constexpr (C == 2) {
    asm volatile(UQ_A8M_PRE "v_mfma_i32_16x16x32_i8 %0, %2, %3, %0\n\tv_mfma_i32_16x16x32_i8 %1, %4, %5, %1" UQ_A8M_POST
                 : "+v"(acc[0]), "+v"(acc[1]) : "v"(av[0]), "v"(bv[0]), "v"(av[1]), "v"(bv[1]));
  } else {
    asm volatile(UQ_A8M_PRE "v_mfma_i32_16x16x32_i8 %0, %4, %5, %0\n\tv_mfma_i32_16x16x32_i8 %1, %6, %7, %1\n\t"
                 "v_mfma_i32_16x16x32_i8 %2, %8, %9, %2\n\tv_mfma_i32_16x16x32_i8 %3, %10, %11, %3" UQ_A8M_POST
                 : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])
                 : "v"(av[0]), "v"(bv[0]), "v"(av[1]), "v"(bv[1]), "v"(av[2]), "v"(bv[2]), "v"(av[3]), "v"(bv[3]));
  }
}
#undef UQ_A8M_PRE
#undef UQ_A8M_POST

// B operand bytes of one MFMA from the lane's 16 codes: INT8 q - 128 as
// signed bytes, INT4 nibbles as bytes (low nibbles, then high, per dword).
template <int S>
__device__ __forceinline__ uint2 a8m_unpack8(const uint8_t* p) {
  if constexpr (S == UQ_INT8) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    return make_uint2(v.x ^ 0x80808080u, v.y ^ 0x80808080u);
  } else if constexpr (S == UQ_INT2) {
    // crumbs c0..c7 of two bytes -> bytes c0 c4 c1 c5 | c2 c6 c3 c7
    const uint32_t h = *reinterpret_cast<const uint16_t*>(p);
    const uint32_t v0 = h & 0x0303u, v1 = (h >> 2) & 0x0303u, v2 = (h >> 4) & 0x0303u, v3 = (h >> 6) & 0x0303u;
    return make_uint2(v0 | (v1 << 16), v2 | (v3 << 16));
  } else {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
    return make_uint2(v & 0x0F0F0F0Fu, (v >> 4) & 0x0F0F0F0Fu);
  }
}
template <int S>
__device__ __forceinline__ uint4 a8m_unpack(const uint8_t* p) {
  if constexpr (S == UQ_INT8) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    return make_uint4(v.x ^ 0x80808080u, v.y ^ 0x80808080u, v.z ^ 0x80808080u, v.w ^ 0x80808080u);
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    return make_uint4(v.x & 0x0F0F0F0Fu, (v.x >> 4) & 0x0F0F0F0Fu, v.y & 0x0F0F0F0Fu, (v.y >> 4) & 0x0F0F0F0Fu);
  }
}

template <int S, int G, int MT, int W, int NBLK>
__global__ __launch_bounds__(64 * W) void gemv_a8_mfma_kernel(const uint8_t* __restrict__ codes,
                                                              const uint8_t* __restrict__ params,
                                                              const uint16_t* __restrict__ x, float* __restrict__ y,
                                                              int n, int k, int m) {
  using Ge = A8mGeo<S, G, MT, W, NBLK>;
  static_assert(Ge::ok, "shape served by the integer matrix-core GEMV");
  constexpr int bits = Ge::bits, KM = Ge::KM, KL = Ge::KL;
  extern __shared__ uint4 lds4[];
  uint8_t* lds = reinterpret_cast<uint8_t*>(lds4);
  int8_t* xs = reinterpret_cast<int8_t*>(lds);                   // [MT][XPITCH] activation codes
  float2* tab = reinterpret_cast<float2*>(lds + Ge::X_BYTES);    // [NG][MT] (s_x, Q as int bits)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint8_t* blk = lds + Ge::X_BYTES + Ge::T_BYTES + wave * (Ge::B_BYTES + Ge::P_BYTES);
  uint8_t* pls = blk + Ge::B_BYTES;

  const int64_t row0 = int64_t(blockIdx.x) * 16;
  const int rowb = k * bits / 8;
  const int ng = k / G;

  // (1) activation loads for quantizing: thread tid takes 16-value pieces
  //     tid, tid + 64 W, ... of the [MT][KP] array (past K or M: zeros; past
  //     the array: a repeat of piece 0, not written).
  constexpr int PIECES = Ge::PIECES;
  uint4 xr[PIECES][2];
#pragma unroll
  for (int i = 0; i < PIECES; ++i) {
    const int p0 = tid + i * 64 * W;
    const int p = p0 < Ge::XPIECES ? p0 : 0;
    const int mm = p / (Ge::KP / 16), k0 = (p % (Ge::KP / 16)) * 16;
    const bool live = mm < m && k0 < k;
    const uint4* src = reinterpret_cast<const uint4*>(x + size_t(live ? mm : 0) * size_t(k) + (live ? k0 : 0));
    xr[i][0] = src[0];
    xr[i][1] = src[1];
    if (!live) xr[i][0] = xr[i][1] = make_uint4(0u, 0u, 0u, 0u);
  }
  __builtin_amdgcn_sched_barrier(0);

  // (2) this wave's parameters (16 rows x QP bytes, 16-byte lanes) and codes
  //     (per block: rows 0-7 then 8-15, eight lanes per 128-byte row piece);
  //     clamped addresses past N or K (their results are not used).
  const int pb0 = wave * Ge::QP;
  constexpr int SPR = Ge::QP / 16;  // 16-byte slots per row
  uint4 pr[Ge::PLOADS];
#pragma unroll
  for (int j = 0; j < Ge::PLOADS; ++j) {
    const int q = j * 64 + lane;
    const int r = q / SPR, o = (q % SPR) * 16;
    int64_t row = row0 + (r < 16 ? r : 15);
    row = row < n ? row : n - 1;
    int off = pb0 + o;
    off = off + 16 <= ng * 4 ? off : ng * 4 - 16;
    pr[j] = load_stream<uint4>(params + row * int64_t(ng) * 4 + off);
  }
  const int lr = lane >> 3, lp = lane & 7;
  uint4 cr[NBLK][2];
#pragma unroll
  for (int b = 0; b < NBLK; ++b)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int64_t row = row0 + 8 * h + lr;
      row = row < n ? row : n - 1;
      int off = wave * Ge::QB + b * kA8mBlock + 16 * lp;
      off = off + 16 <= rowb ? off : rowb - 16;
      cr[b][h] = load_stream<uint4>(codes + row * int64_t(rowb) + off);
    }
  __builtin_amdgcn_sched_barrier(0);

  // (3) quantize: max |x| over the group's G / 16 consecutive lanes, codes
  //     rint(x * fp32(127 / a)) clamped to +-127 (the same steps as the
  //     dot-product A8 kernel), written in the B byte order; Q summed the
  //     same way (exact integers); (s_x, Q) per (group, row).
#pragma unroll
  for (int i = 0; i < PIECES; ++i) {
    const int p0 = tid + i * 64 * W;
    const bool here = p0 < Ge::XPIECES;  // uniform over a group's lanes
    const int p = here ? p0 : 0;
    const int mm = p / (Ge::KP / 16), k0 = (p % (Ge::KP / 16)) * 16;
    float v[16];
    float a = unpack16(xr[i][0], xr[i][1], v);
    a = group_max<G>(a);
    uint32_t packed[4];
    int qs;
    quantize_piece<S>(v, a, packed, qs);
#pragma unroll
    for (int off = 1; off < G / 16; off <<= 1) qs += __shfl_xor(qs, off, 64);
    if (here) *reinterpret_cast<uint4*>(xs + mm * Ge::XPITCH + k0) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    if (here && (p % (G / 16)) == 0) tab[(k0 / G) * MT + mm] = make_float2(a / 127.0f, __int_as_float(qs));
  }

  // (4) this wave's parameters into its LDS rows
#pragma unroll
  for (int j = 0; j < Ge::PLOADS; ++j) {
    const int q = j * 64 + lane;
    const int r = q / SPR, o = (q % SPR) * 16;
    if (r < 16) *reinterpret_cast<uint4*>(pls + r * Ge::PP + o) = pr[j];
  }
  __syncthreads();

  // (5) blocks: move the two dense loads into the MFMA layout through LDS,
  //     then per group its MFMA chain and its scaling.
  const int ln = lane & 15, lg = lane >> 4;          // MFMA column (weight row) and k block of this lane
  const int8_t* xa = xs + (ln % MT) * Ge::XPITCH;     // this lane's A row (rows past MT repeat)
  const uint8_t* bp = blk + ln * kA8mRowPitch;        // this lane's weight row of the block
  f32x4 yacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int b = 0; b < NBLK; ++b) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      *reinterpret_cast<uint4*>(blk + (8 * h + lr) * kA8mRowPitch + 16 * lp) = cr[b][h];
    // (a wave's LDS accesses execute in issue order: only the compiler must
    //  not move the block's reads and writes across each other)
    asm volatile("" ::: "memory");
    constexpr int GPB = Ge::GPB;  // groups per block (a group never straddles blocks)
    static_assert(Ge::HALF || Ge::MPB % Ge::MPG == 0, "blocks hold whole groups");
    constexpr int SBG = GPB < 4 ? GPB : 4;  // groups per sub-block
    static_assert(GPB % SBG == 0, "sub-blocks hold whole groups");
    using Frag = typename std::conditional<KM == 64, uint4, uint2>::type;
#pragma unroll
    for (int sbk = 0; sbk < GPB / SBG; ++sbk) {
      if constexpr (GPB / SBG > 1) {
        // one sub-block's reads in flight at a time
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
      // the sub-block's groups: operands first, then their chains (one-MFMA
      // chains in one asm statement: measured on MI355X, INT4 G64 N11008 M=2
      // / 4 / 8 8.7 / 10.3 / 13.1 -> 8.1 / 9.8 / 12.7 us), then each group's
      // scaling
      Frag av[SBG][Ge::MPG], bv[SBG][Ge::MPG];
      float sx[SBG][4];
      int qs[SBG][4];
      uint32_t par[SBG];
#pragma unroll
      for (int g = 0; g < SBG; ++g) {
        const int gb = sbk * SBG + g;                             // group within the block
        const int q0 = Ge::HALF ? gb / 2 : gb * Ge::MPG;          // its (first) k range in the block
        const int kq0 = wave * Ge::QK + (b * Ge::MPB + q0) * KM;  // that range's first k
        const int gk = kq0 / G + (Ge::HALF ? gb % 2 : 0);         // global group
        const int gi = b * GPB + gb;                              // group within the wave
#pragma unroll
        for (int jj = 0; jj < Ge::MPG; ++jj) {
          const int q = q0 + jj;
          if constexpr (Ge::HALF) {
            // the range's other group: its lanes' B bytes zeroed
            const uint2 v = a8m_unpack8<S>(bp + (q * KM + KL * lg) * bits / 8);
            const bool mine = (lg >> 1) == (gb % 2);
            bv[g][jj] = make_uint2(mine ? v.x : 0u, mine ? v.y : 0u);
            av[g][jj] = *reinterpret_cast<const uint2*>(xa + kq0 + KL * lg);
          } else if constexpr (KM == 64) {
            bv[g][jj] = a8m_unpack<S>(bp + (q * KM + KL * lg) * bits / 8);
            av[g][jj] = *reinterpret_cast<const uint4*>(xa + kq0 + jj * KM + KL * lg);
          } else {
            bv[g][jj] = a8m_unpack8<S>(bp + (q * KM + KL * lg) * bits / 8);
            av[g][jj] = *reinterpret_cast<const uint2*>(xa + kq0 + jj * KM + KL * lg);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float2 t = tab[gk * MT + (4 * lg + i) % MT];
          sx[g][i] = t.x;
          qs[g][i] = __float_as_int(t.y);
        }
        par[g] = gk < ng ? *reinterpret_cast<const uint32_t*>(pls + ln * Ge::PP + gi * 4) : 0u;  // past K: 0
      }
      i32x4v acc[SBG];
#pragma unroll
      for (int g = 0; g < SBG; ++g) acc[g] = i32x4v{0, 0, 0, 0};
      if constexpr (Ge::MPG == 1 && (SBG == 2 || SBG == 4)) {
        Frag a1[SBG], b1[SBG];
#pragma unroll
        for (int g = 0; g < SBG; ++g) {
          a1[g] = av[g][0];
          b1[g] = bv[g][0];
        }
        if constexpr (KM == 64) a8_chains1<SBG>(acc, a1, b1);
        else a8_chains32<SBG>(acc, a1, b1);
      } else {  // two-MFMA chains (128-code groups): sharing one statement measured no faster
        static_assert(KM == 64, "32-code groups: one MFMA each");
#pragma unroll
        for (int g = 0; g < SBG; ++g) a8_chain<Ge::MPG>(acc[g], av[g], bv[g]);
      }
#pragma unroll
      for (int g = 0; g < SBG; ++g) {
        const float sc = h2f(uint16_t(par[g] & 0xFFFFu)), zc = h2f(uint16_t(par[g] >> 16));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int dd = S == UQ_INT8 ? acc[g][i] + 128 * qs[g][i] : acc[g][i];
          const float t = __builtin_fmaf(sc, float(dd), zc * float(qs[g][i]));
          yacc[i] = __builtin_fmaf(sx[g][i], t, yacc[i]);
        }
        // with several sub-blocks per block (16- and 32-code groups) the
        // scaling stays with its chain (left free, the compiler moves it past
        // the last chain and spills: 256 VGPRs and scratch)
        asm volatile("" : "+v"(yacc));
      }
    }
    asm volatile("" ::: "memory");  // the next block's writes stay after this block's reads
  }

  // (6) add the W partial tiles in wave order and store y[m][row] for m < M
  __syncthreads();
  *reinterpret_cast<f32x4*>(lds + Ge::X_BYTES + Ge::T_BYTES + wave * (Ge::B_BYTES + Ge::P_BYTES) + lane * 16) = yacc;
  __syncthreads();
  if (wave != 0) return;
  f32x4 sum = yacc;
#pragma unroll
  for (int w = 1; w < W; ++w) {
    const f32x4 v =
        *reinterpret_cast<const f32x4*>(lds + Ge::X_BYTES + Ge::T_BYTES + w * (Ge::B_BYTES + Ge::P_BYTES) + lane * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) sum[i] += v[i];
  }
  const int64_t row = row0 + ln;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int mm = 4 * lg + i;
    if (mm < m && row < n) y[size_t(mm) * size_t(n) + size_t(row)] = sum[i];
  }
}

// Blocks per wave, rounded up to 1, 2, 4 or 8 (the block loop is unrolled); 0 past 8.
inline int a8m_nblk(int64_t rowb, int w) {
  const int64_t nb = (rowb + w * kA8mBlock - 1) / (w * kA8mBlock);
  return nb <= 1 ? 1 : nb <= 2 ? 2 : nb <= 4 ? 4 : nb <= 8 ? 8 : 0;
}

// Whether the shape runs on the integer matrix cores: whole 16-byte parameter
// slots per row and per wave, the staged codes within their LDS budget.
template <int S, int G>
bool a8m_fits(int64_t k, int mt, int w) {
  constexpr int bits = Fmt<S>::bits;
  const int nb = a8m_nblk(k * bits / 8, w);
  if (!nb) return false;
  const int64_t kp = int64_t(nb) * w * kA8mBlock * 8 / bits;
  const int64_t qp = kp / w / G * 4;
  return a8_mfma_scheme<S, G>() && int64_t(mt) * (kp + 16) <= kA8mXBytes && (k / G) % 4 == 0 && qp % 16 == 0 &&
         (kp / w) % G == 0;
}

template <int S, int G, int MT, int W, int NBLK>
hipError_t launch_a8m_t(const uq_layout* L, const void* codes, const void* params, const uint16_t* x, float* y,
                        int m, hipStream_t stream) {
  using Ge = A8mGeo<S, G, MT, W, NBLK>;
  if constexpr (!Ge::ok) {
    return hipErrorInvalidValue;  // never chosen: a8m_fits() rules the shape out
  } else {
    const int n = int(L->n), k = int(L->k);
    const int64_t blocks = (int64_t(n) + 15) / 16;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const uint8_t* c8 = static_cast<const uint8_t*>(codes);
    const uint8_t* p8 = static_cast<const uint8_t*>(params);
    int nn = n, kk = k, mm = m;
    void* args[] = {&c8, &p8, (void*)&x, &y, &nn, &kk, &mm};
    return hipLaunchKernel(reinterpret_cast<const void*>(&gemv_a8_mfma_kernel<S, G, MT, W, NBLK>),
                           dim3(unsigned(blocks)), dim3(64 * W), args, size_t(Ge::LDS), stream);
  }
}

template <int S, int G, int MT, int W>
hipError_t launch_a8m_w(const uq_layout* L, const void* codes, const void* params, const uint16_t* x, float* y,
                        int m, hipStream_t stream) {
  switch (a8m_nblk(L->k * Fmt<S>::bits / 8, W)) {
    case 1: return launch_a8m_t<S, G, MT, W, 1>(L, codes, params, x, y, m, stream);
    case 2: return launch_a8m_t<S, G, MT, W, 2>(L, codes, params, x, y, m, stream);
    case 4: return launch_a8m_t<S, G, MT, W, 4>(L, codes, params, x, y, m, stream);
    case 8: return launch_a8m_t<S, G, MT, W, 8>(L, codes, params, x, y, m, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace uq
