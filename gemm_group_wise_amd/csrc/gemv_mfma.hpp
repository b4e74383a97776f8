// Fused group-wise dequant + GEMV on the fp16 matrix cores, for 2 to 8
// activation rows ("Ultra LLM Engine", Core Components > Fused Kernels:
// dequantized-weight GEMV during decode; Highlights, Batching: a batch of
// decode rows shares one pass over the weights).
//
// With several activation rows the dot-product GEMV spends about half a
// VALU instruction per weight per activation row on v_dot2; here the
// products run on v_mfma_f32_16x16x32_f16 (16x16x16 for INT2, whose groups
// are 16 codes) and the VALU cost per weight no longer grows with M.
// The products are exact and accumulate in fp32, as in the dot-product
// GEMV:
//   * B operand: each code as the exact fp16 1024 + q (0x6400 | q, one
//     v_and_or_b32 per pair of codes; INT8 one v_perm_b32 per pair);
//   * A operand: x in fp16, exactly as given (rows past M repeat real rows:
//     computed, never stored);
//   * per weight group g, the MFMA chain starts from C = -1024 * SX (SX = the
//     group's sum of x, fp32) so that it ends at t = sum q * x; then
//     y += s * t + z * SX, which is sum x * (q * s + z).
// MFMA lane layout (16x16xK): lane l holds A[row l % 16][k-block l / 16],
// B[k-block l / 16][column l % 16] and D[rows 4 (l / 16) .. + 3][column l % 16].
// Columns are 16 weight rows, rows are activation rows.  Within an MFMA the
// assignment of k to (lane block, element) is free as long as A and B agree:
// each scheme's unpacked pair order is matched by the order in which its
// activations are staged.
//
// Work split: a workgroup of W waves owns 16 weight rows; wave w takes the
// w-th of W equal slices of every row's code bytes (whole 128-byte blocks).
// Codes are loaded densely (eight rows x 128 bytes per wave instruction, full
// cache lines), all at once, then moved through a per-wave LDS block into the
// MFMA layout; a wave's parameters (up to 32 bytes per row) are loaded by
// each lane for its own weight row and stay in registers (longer parameter
// rows go through LDS like the codes).  x is staged in LDS once per workgroup
// with the per-group sums.  The W partial 16 x 16 tiles are added in a fixed
// order through LDS at the end (bitwise repeatable).
#pragma once

#include "device_common.hpp"

namespace uq {
namespace {

typedef _Float16 f16x8v __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4v __attribute__((ext_vector_type(4)));

// k per MFMA; codes a lane of an MFMA uses sit in one dword (INT4: 8 codes;
// INT2: the 16-code group's dword, of which it takes 4) or two (INT8).
template <int S> struct Mf;
template <> struct Mf<UQ_INT4> { static constexpr int KM = 32; };
template <> struct Mf<UQ_INT8> { static constexpr int KM = 32; };
template <> struct Mf<UQ_INT2> { static constexpr int KM = 16; };

constexpr int kMfBlock = 128;          // code bytes per row per block (two dense loads of 8 rows)
constexpr int kMfXBytes = 64 * 1024;   // most LDS the staged activations may take

// Schemes and groups the matrix-core GEMV serves (16x16x32 MFMAs, chains of
// one to four MFMAs per group; INT2 with 16-code groups one 16x16x16 MFMA
// per group); INT2 with longer groups keeps the dot-product kernel.
template <int S, int G>
constexpr bool mfma_gemv_scheme() {
  return (S == UQ_INT4 && (G == 32 || G == 64 || G == 128)) || (S == UQ_INT8 && (G == 32 || G == 64 || G == 128)) ||
         (S == UQ_INT2 && G == 16);
}

template <int S, int G, int MT, int W, int NBLK>
struct MfGeo {
  static constexpr int bits = Fmt<S>::bits;
  static constexpr int KM = Mf<S>::KM;
  static constexpr int QB = NBLK * kMfBlock;                 // code bytes per row per wave
  static constexpr int QK = QB * 8 / bits;                   // k per wave
  static constexpr int KP = W * QK;                          // padded K of a launch
  static constexpr int GPW = QK / G;                         // groups per wave
  static constexpr int NG = KP / G;                          // groups of the padded K
  static constexpr int MPB = kMfBlock * 8 / bits / KM;       // MFMAs per block
  static constexpr int MPG = G / KM;                         // MFMAs per group
  static constexpr int QP = GPW * 4;                         // parameter bytes per row per wave
  static constexpr int PP = QP + 16;                         // their LDS pitch per row
  static constexpr int XPITCH = KP * 2 + 16;                 // LDS bytes per staged activation row
  static constexpr int X_BYTES = MT * XPITCH;
  static constexpr int T_BYTES = MT * NG * 8;                // (-1024 * SX, SX) per (group, row)
  // With eight staged activation rows, INT4 with its parameters in registers
  // stages each block in two halves of 64 bytes per row, one per four-MFMA
  // sub-block, so that two workgroups fit a CU (80,000 bytes of LDS; measured
  // on MI355X, INT4 G64 N11008 M=8 13.6 -> 11.4 us, N14336 17.5 -> 14.0 us;
  // with fewer rows the whole blocks measured faster: M=2 / 4 8.5 / 9.3
  // against 9.3 / 10.0 us, the half-line code loads costing more than the
  // occupancy they no longer buy).
  static constexpr int HB = (bits == 4 && QP <= 32 && MT == 8) ? 2 : 1;
  static constexpr int BPITCH = kMfBlock / HB + 16;          // LDS bytes per row (16-byte reads: distinct banks)
  static constexpr int B_BYTES = 16 * BPITCH;                // one wave's block (or half block)
  // A wave's parameters: up to two 16-byte slots per row go straight into
  // each lane's registers (the lane's weight row; the four lanes of a row
  // load the same bytes), which keeps them out of LDS so that more
  // workgroups fit a CU; longer rows of parameters (INT2 G16: 32 groups per
  // wave) go through a per-wave LDS area.
  static constexpr bool PREG = QP <= 32;
  static constexpr int PR = PREG ? QP / 16 : 1;              // 16-byte parameter loads per lane (registers)
  static constexpr int P_BYTES = PREG ? 0 : 16 * PP;         // one wave's parameters in LDS
  static constexpr int LDS = X_BYTES + T_BYTES + W * (B_BYTES + P_BYTES);
  static constexpr int PLOADS = (16 * QP + 1023) / 1024;     // 16-byte parameter loads per lane (LDS)
  static constexpr int XPIECES = MT * KP / 16;               // 16-activation pieces staged
  static constexpr int PIECES = (XPIECES + 64 * W - 1) / (64 * W);  // per thread
  // An MFMA lies in one group and a wave holds whole groups; a wave's
  // parameters are whole 16-byte slots per row; a group's staged pieces are
  // consecutive lanes of one wave; the activations fit their LDS budget.
  static constexpr bool ok = mfma_gemv_scheme<S, G>() && G % KM == 0 && QK % G == 0 && QP % 16 == 0 &&
                             G / 16 <= 64 && 64 % (G / 16) == 0 && MT * KP * 2 <= kMfXBytes &&
                             LDS <= 160 * 1024;
};

// Stage order of 16 consecutive activations for a scheme (position -> source
// index), matching the order the unpacked codes take in the B operand.
template <int S>
__device__ __forceinline__ constexpr int mf_src(int p) {
  if constexpr (S == UQ_INT4) {
    const int e = p & 7;  // pairs (q0,q4)(q1,q5)(q2,q6)(q3,q7) of each 8
    return (p & 8) + (e >> 1) + 4 * (e & 1);
  } else if constexpr (S == UQ_INT2) {
    // lane block g of a 16-code MFMA takes codes g, g + 8, g + 4, g + 12
    const int g = p >> 2, e = p & 3;
    return g + 8 * (e & 1) + 4 * (e >> 1);
  } else {
    return p;
  }
}

// B operand of one MFMA from the lane's code dword(s): pairs of fp16 1024 + q.
template <int S>
__device__ __forceinline__ void mf_unpack(uint32_t d0, uint32_t d1, int lg, uint32_t (&b)[4]) {
  const uint32_t magic = kMagic2;
  if constexpr (S == UQ_INT2) {
    // the group's dword holds codes c0..c15 (crumb i at bit 2i); lane block
    // lg takes (c_lg, c_lg+8) and (c_lg+4, c_lg+12): bits 2 lg and 2 lg + 8
    // of each half
    b[0] = and_or(d0 >> (2 * lg), 0x00030003u, magic);
    b[1] = and_or(d0 >> (2 * lg + 8), 0x00030003u, magic);
    b[2] = 0u;
    b[3] = 0u;
  } else if constexpr (S == UQ_INT4) {
    b[0] = and_or(d0, 0x000F000Fu, magic);
    b[1] = and_or(d0 >> 4, 0x000F000Fu, magic);
    b[2] = and_or(d0 >> 8, 0x000F000Fu, magic);
    b[3] = and_or(d0 >> 12, 0x000F000Fu, magic);
  } else {  // INT8
    b[0] = __builtin_amdgcn_perm(magic, d0, 0x05010500u);
    b[1] = __builtin_amdgcn_perm(magic, d0, 0x05030502u);
    b[2] = __builtin_amdgcn_perm(magic, d1, 0x05010500u);
    b[3] = __builtin_amdgcn_perm(magic, d1, 0x05030502u);
  }
}

// Each group's MFMA chain is one inline-asm statement: the accumulator is
// tied to the destination, the wait states are explicit, and nothing can
// come between an MFMA and the point where the accumulator is read.  Left to
// itself, the compiler produced (for some instantiations) untied
// accumulations, destinations overlapping the A / B registers and an
// accumulator spilled to scratch a few cycles after its MFMA; those
// instantiations returned wrong values in some lanes on the GPU, while the
// same source with s_nop padding around every MFMA was correct.  Here:
// sixteen wait states before each MFMA (its operands were just written by
// VALU or LDS, or it adds to the previous MFMA's result) and 21 after the
// last one before the accumulator is read (more than the MFMA's passes).
#define UQ_MF_PRE "s_nop 7\n\ts_nop 7\n\t"
#define UQ_MF_OP "v_mfma_f32_16x16x32_f16 "
#define UQ_MF_POST "\n\ts_nop 7\n\ts_nop 7\n\ts_nop 4"
template <int N>
__device__ __forceinline__ void mfma_chain(f32x4& acc, const f16x8v (&a)[N], const f16x8v (&b)[N]) {
  static_assert(N == 1 || N == 2 || N == 4, "chains of 1, 2 or 4 MFMAs");
  if constexpr (N == 1) {
    asm volatile(UQ_MF_PRE UQ_MF_OP "%0, %1, %2, %0" UQ_MF_POST : "+v"(acc) : "v"(a[0]), "v"(b[0]));
  } else if constexpr (N == 2) {
    asm volatile(UQ_MF_PRE UQ_MF_OP "%0, %1, %2, %0\n\t" UQ_MF_PRE UQ_MF_OP "%0, %3, %4, %0" UQ_MF_POST
                 : "+v"(acc) : "v"(a[0]), "v"(b[0]), "v"(a[1]), "v"(b[1]));
  } else {
    asm volatile(UQ_MF_PRE UQ_MF_OP "%0, %1, %2, %0\n\t" UQ_MF_PRE UQ_MF_OP "%0, %3, %4, %0\n\t"
                 UQ_MF_PRE UQ_MF_OP "%0, %5, %6, %0\n\t" UQ_MF_PRE UQ_MF_OP "%0, %7, %8, %0" UQ_MF_POST
                 : "+v"(acc) : "v"(a[0]), "v"(b[0]), "v"(a[1]), "v"(b[1]), "v"(a[2]), "v"(b[2]), "v"(a[3]), "v"(b[3]));
  }
}
// Several groups' chains in one statement, independent accumulators
// interleaved: the wait states before the first MFMA, between the dependent
// MFMAs of a chain and after the last are paid once for all of them (each
// dependent MFMA still has sixteen or more wait states after the one it
// adds to; the operands were all written before the statement).
template <int C>
__device__ __forceinline__ void mfma_chains1(f32x4 (&acc)[C], const f16x8v (&a)[C], const f16x8v (&b)[C]) {
  static_assert(C == 2 || C == 4, "two or four one-MFMA chains");
  if constexpr (C == 2) {
    asm volatile(UQ_MF_PRE UQ_MF_OP "%0, %2, %3, %0\n\t" UQ_MF_OP "%1, %4, %5, %1" UQ_MF_POST
                 : "+v"(acc[0]), "+v"(acc[1]) : "v"(a[0]), "v"(b[0]), "v"(a[1]), "v"(b[1]));
  } else {
    asm volatile(UQ_MF_PRE UQ_MF_OP "%0, %4, %5, %0\n\t" UQ_MF_OP "%1, %6, %7, %1\n\t" UQ_MF_OP "%2, %8, %9, %2\n\t"
                 UQ_MF_OP "%3, %10, %11, %3" UQ_MF_POST
                 : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])
                 : "v"(a[0]), "v"(b[0]), "v"(a[1]), "v"(b[1]), "v"(a[2]), "v"(b[2]), "v"(a[3]), "v"(b[3]));
  }
}
// Two chains of two MFMAs: a0 b0 of each, then a1 b1 of each.
__device__ __forceinline__ void mfma_chains2x2(f32x4 (&acc)[2], const f16x8v (&a)[2][2], const f16x8v (&b)[2][2]) {
  asm volatile(UQ_MF_PRE UQ_MF_OP "%0, %2, %3, %0\n\t" UQ_MF_OP "%1, %6, %7, %1\n\t"
               UQ_MF_PRE UQ_MF_OP "%0, %4, %5, %0\n\t" UQ_MF_OP "%1, %8, %9, %1" UQ_MF_POST
               : "+v"(acc[0]), "+v"(acc[1])
               : "v"(a[0][0]), "v"(b[0][0]), "v"(a[0][1]), "v"(b[0][1]), "v"(a[1][0]), "v"(b[1][0]), "v"(a[1][1]),
                 "v"(b[1][1]));
}
// INT2: eight 16-code groups, one v_mfma_f32_16x16x16_f16 each (4 fp16 per lane).
__device__ __forceinline__ void mfma_chains16x8(f32x4 (&acc)[8], const f16x4v (&a)[8], const f16x4v (&b)[8]) {
  asm volatile(UQ_MF_PRE "v_mfma_f32_16x16x16_f16 %0, %8, %9, %0\n\tv_mfma_f32_16x16x16_f16 %1, %10, %11, %1\n\t"
               "v_mfma_f32_16x16x16_f16 %2, %12, %13, %2\n\tv_mfma_f32_16x16x16_f16 %3, %14, %15, %3\n\t"
               "v_mfma_f32_16x16x16_f16 %4, %16, %17, %4\n\tv_mfma_f32_16x16x16_f16 %5, %18, %19, %5\n\t"
               "v_mfma_f32_16x16x16_f16 %6, %20, %21, %6\n\tv_mfma_f32_16x16x16_f16 %7, %22, %23, %7" UQ_MF_POST
               : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]), "+v"(acc[6]), "+v"(acc[7])
               : "v"(a[0]), "v"(b[0]), "v"(a[1]), "v"(b[1]), "v"(a[2]), "v"(b[2]), "v"(a[3]), "v"(b[3]),
                 "v"(a[4]), "v"(b[4]), "v"(a[5]), "v"(b[5]), "v"(a[6]), "v"(b[6]), "v"(a[7]), "v"(b[7]));
}
#undef UQ_MF_PRE
#undef UQ_MF_OP
#undef UQ_MF_POST

template <int S, int G, int MT, int W, int NBLK>
__global__ __launch_bounds__(64 * W) void gemv_mfma_kernel(const uint8_t* __restrict__ codes,
                                                           const uint8_t* __restrict__ params,
                                                           const uint16_t* __restrict__ x, float* __restrict__ y,
                                                           int n, int k, int m) {
  using Ge = MfGeo<S, G, MT, W, NBLK>;
  static_assert(Ge::ok, "shape served by the matrix-core GEMV");
  constexpr int bits = Ge::bits, KM = Ge::KM;
  extern __shared__ uint4 lds4[];
  uint8_t* lds = reinterpret_cast<uint8_t*>(lds4);
  uint8_t* xs = lds;                                            // [MT][XPITCH] staged activations
  float2* tab = reinterpret_cast<float2*>(lds + Ge::X_BYTES);   // [NG][MT] (-1024 SX, SX)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint8_t* blk = lds + Ge::X_BYTES + Ge::T_BYTES + wave * (Ge::B_BYTES + Ge::P_BYTES);
  uint8_t* pls = blk + Ge::B_BYTES;

  const int64_t row0 = int64_t(blockIdx.x) * 16;
  const int rowb = k * bits / 8;
  const int ng = k / G;

  // (1) activation loads for staging: thread tid takes 16-value pieces
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
  // (parameter rows are whole 16-byte slots: ng % 4 == 0, checked at launch;
  //  slots past the row's groups load a valid slot and are never used)
  const int pb0 = wave * Ge::QP;  // first parameter byte of the wave in a row
  constexpr int SPR = Ge::QP / 16;  // 16-byte slots per row
  uint4 pr[Ge::PREG ? Ge::PR : Ge::PLOADS];
  if constexpr (Ge::PREG) {
    int64_t row = row0 + (lane & 15);
    row = row < n ? row : n - 1;
#pragma unroll
    for (int j = 0; j < Ge::PR; ++j) {
      int off = pb0 + 16 * j;
      off = off + 16 <= ng * 4 ? off : ng * 4 - 16;
      pr[j] = load_stream<uint4>(params + row * int64_t(ng) * 4 + off);
    }
  } else {
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
  }
  // Dense code loads, two per block: rows 0-7 then 8-15 (lane: row within
  // eight, 16-byte piece of the 128 bytes), or with half blocks the first then
  // the second 64 bytes of all 16 rows (lane: row, 16-byte piece of the half).
  const int lr = Ge::HB == 1 ? lane >> 3 : lane >> 2, lp = Ge::HB == 1 ? lane & 7 : lane & 3;
  uint4 cr[NBLK][2];
#pragma unroll
  for (int b = 0; b < NBLK; ++b)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int64_t row = row0 + (Ge::HB == 1 ? 8 * h + lr : lr);
      row = row < n ? row : n - 1;
      int off = wave * Ge::QB + b * kMfBlock + (Ge::HB == 1 ? 16 * lp : 64 * h + 16 * lp);
      off = off + 16 <= rowb ? off : rowb - 16;
      cr[b][h] = load_stream<uint4>(codes + row * int64_t(rowb) + off);
    }
  __builtin_amdgcn_sched_barrier(0);

  // (3) stage: reorder each 16 activations for the scheme's pair order and
  //     sum each group (fp32, fixed order: 16-value partial sums, then a lane
  //     reduction over the G / 16 consecutive lanes of a group).
#pragma unroll
  for (int i = 0; i < PIECES; ++i) {
    const int p0 = tid + i * 64 * W;
    const bool here = p0 < Ge::XPIECES;  // uniform over a group's lanes (whole groups per wave pass)
    const int p = here ? p0 : 0;
    const int mm = p / (Ge::KP / 16), k0 = (p % (Ge::KP / 16)) * 16;
    uint16_t v[16];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t d = dword_of(xr[i][e >> 2], e & 3);
      v[2 * e] = uint16_t(d & 0xFFFFu);
      v[2 * e + 1] = uint16_t(d >> 16);
    }
    uint32_t o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      o[e] = uint32_t(v[mf_src<S>(2 * e)]) | (uint32_t(v[mf_src<S>(2 * e + 1)]) << 16);
    uint4* dst = reinterpret_cast<uint4*>(xs + mm * Ge::XPITCH + k0 * 2);
    if (here) {
      dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
    const f16x2 one2 = {_Float16(1.0f), _Float16(1.0f)};
    float sx = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sx = __builtin_amdgcn_fdot2(as_h2(dword_of(xr[i][e >> 2], e & 3)), one2, sx, false);
    // group sum over G / 16 consecutive lanes (pieces of one group are consecutive p)
#pragma unroll
    for (int off = 1; off < G / 16; off <<= 1) sx += __shfl_xor(sx, off, 64);
    if (here && (p % (G / 16)) == 0) tab[(k0 / G) * MT + mm] = make_float2(-1024.0f * sx, sx);
  }

  // (4) this wave's parameters into its LDS rows
  if constexpr (!Ge::PREG) {
#pragma unroll
    for (int j = 0; j < Ge::PLOADS; ++j) {
      const int q = j * 64 + lane;
      const int r = q / SPR, o = (q % SPR) * 16;
      if (r < 16) *reinterpret_cast<uint4*>(pls + r * Ge::PP + o) = pr[j];
    }
  }
  __syncthreads();

  // (5) blocks: move the two dense loads into the MFMA layout through LDS,
  //     then the block in sub-blocks of up to four MFMAs: every LDS read
  //     of a sub-block first (one wait), then per group its MFMA chain and
  //     its scaling.
  const int ln = lane & 15, lg = lane >> 4;   // MFMA column (weight row) and k block of this lane
  const uint8_t* xa = xs + (ln % MT) * Ge::XPITCH;  // this lane's A row (rows past MT repeat)
  const uint8_t* bp = blk + ln * Ge::BPITCH;        // this lane's weight row of the block
  // MFMAs per sub-block: four (67-90 VGPRs up to eight activation rows;
  // eight MFMAs per sub-block took 128 and left two workgroups per CU); INT2
  // G16, which runs five to eight rows at one workgroup per CU (its staged
  // activations and per-group sums take 82 KB of LDS), eight, one per group
  // (118-162 VGPRs; measured on MI355X, N4096 M=8 7.2 -> 7.0 us)
  constexpr int SB = KM == 16 ? 8 : (Ge::MPB < 4 ? Ge::MPB : 4);
  constexpr int GS = SB / Ge::MPG;                  // groups per sub-block
  static_assert(Ge::MPB % SB == 0 && SB % Ge::MPG == 0, "sub-blocks hold whole groups");
  static_assert(Ge::HB == 1 || Ge::MPB / SB == Ge::HB, "a half block per sub-block");
  f32x4 yacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int b = 0; b < NBLK; ++b) {
    if constexpr (Ge::HB == 1) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        *reinterpret_cast<uint4*>(blk + (8 * h + lr) * Ge::BPITCH + 16 * lp) = cr[b][h];
    }
    // (a wave's LDS accesses execute in issue order: only the compiler must
    //  not move the block's reads and writes across each other)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int sb = 0; sb < Ge::MPB / SB; ++sb) {
      if constexpr (Ge::MPB / SB > 1) {
        // one sub-block's reads in flight at a time (left free, the compiler
        // hoists every sub-block's LDS reads and runs out of registers)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (Ge::HB == 2) {
        // this sub-block's half of the block (written after the previous
        // sub-block's reads, which a wave's LDS accesses keep in order)
        *reinterpret_cast<uint4*>(blk + lr * Ge::BPITCH + 16 * lp) = cr[b][sb];
        asm volatile("" ::: "memory");
      }
      const int q0 = sb * SB;                                   // first MFMA of the sub-block in the block
      const int kq0 = wave * Ge::QK + (b * Ge::MPB + q0) * KM;  // its first k
      const int gi0 = (b * Ge::MPB + q0) / Ge::MPG;             // its first group within the wave
      // B dwords, A fragments, the groups' (-1024 SX, SX) rows and parameters
      uint32_t bd[SB][2];
      uint4 av[SB];
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        const int q = q0 + j;
        if constexpr (S == UQ_INT2) {
          bd[j][0] = *reinterpret_cast<const uint32_t*>(bp + q * 4);  // the group's 16 codes
          bd[j][1] = 0u;
        } else if constexpr (S == UQ_INT4) {
          bd[j][0] = *reinterpret_cast<const uint32_t*>(bp + (q % (Ge::MPB / Ge::HB)) * 16 + 4 * lg);
          bd[j][1] = 0u;
        } else {
          const uint2 v = *reinterpret_cast<const uint2*>(bp + q * 32 + 8 * lg);
          bd[j][0] = v.x;
          bd[j][1] = v.y;
        }
        if constexpr (KM == 16) {
          const uint2 t = *reinterpret_cast<const uint2*>(xa + (kq0 + j * KM + 4 * lg) * 2);
          av[j] = make_uint4(t.x, t.y, 0u, 0u);
        } else {
          av[j] = *reinterpret_cast<const uint4*>(xa + (kq0 + j * KM + 8 * lg) * 2);
        }
      }
      float tc[GS][4], ts[GS][4];
      uint32_t par[GS];
#pragma unroll
      for (int g = 0; g < GS; ++g) {
        const int gk = kq0 / G + g;  // global group
        const float2* t = tab + gk * MT;
        if constexpr (MT >= 4) {
          const float4 lo = *reinterpret_cast<const float4*>(t + ((4 * lg) % MT));
          const float4 hi = *reinterpret_cast<const float4*>(t + ((4 * lg) % MT) + 2);
          tc[g][0] = lo.x; ts[g][0] = lo.y; tc[g][1] = lo.z; ts[g][1] = lo.w;
          tc[g][2] = hi.x; ts[g][2] = hi.y; tc[g][3] = hi.z; ts[g][3] = hi.w;
        } else if constexpr (MT == 2) {
          const float4 v = *reinterpret_cast<const float4*>(t);
          tc[g][0] = tc[g][2] = v.x; ts[g][0] = ts[g][2] = v.y;
          tc[g][1] = tc[g][3] = v.z; ts[g][1] = ts[g][3] = v.w;
        } else {
          const float2 v = t[0];
#pragma unroll
          for (int i = 0; i < 4; ++i) { tc[g][i] = v.x; ts[g][i] = v.y; }
        }
        uint32_t pv;
        if constexpr (Ge::PREG) pv = dword_of(pr[(gi0 + g) / 4], (gi0 + g) % 4);
        else pv = *reinterpret_cast<const uint32_t*>(pls + ln * Ge::PP + (gi0 + g) * 4);
        par[g] = gk < ng ? pv : 0u;  // past K: 0
      }
      // every group's chain starts at -1024 * SX; the sub-block's chains run
      // in one asm statement where a helper covers the shape
      f32x4 acc[GS];
#pragma unroll
      for (int g = 0; g < GS; ++g) acc[g] = f32x4{tc[g][0], tc[g][1], tc[g][2], tc[g][3]};
      if constexpr (KM == 16) {
        static_assert(Ge::MPG == 1 && GS == 8, "16-code groups: one MFMA each, eight per sub-block");
        f16x4v ca[8], cb[8];
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          uint32_t bb[4];
          mf_unpack<S>(bd[g][0], bd[g][1], lg, bb);
          ca[g] = __builtin_bit_cast(f16x4v, make_uint2(av[g].x, av[g].y));
          cb[g] = __builtin_bit_cast(f16x4v, make_uint2(bb[0], bb[1]));
        }
        mfma_chains16x8(acc, ca, cb);
      } else {
        f16x8v ca[GS][Ge::MPG], cb[GS][Ge::MPG];
#pragma unroll
        for (int g = 0; g < GS; ++g)
#pragma unroll
          for (int jj = 0; jj < Ge::MPG; ++jj) {
            const int j = g * Ge::MPG + jj;
            uint32_t bb[4];
            mf_unpack<S>(bd[j][0], bd[j][1], lg, bb);
            ca[g][jj] = __builtin_bit_cast(f16x8v, av[j]);
            cb[g][jj] = __builtin_bit_cast(f16x8v, make_uint4(bb[0], bb[1], bb[2], bb[3]));
          }
        if constexpr (Ge::MPG == 1 && (GS == 2 || GS == 4)) {
          f16x8v a1[GS], b1[GS];
#pragma unroll
          for (int g = 0; g < GS; ++g) {
            a1[g] = ca[g][0];
            b1[g] = cb[g][0];
          }
          mfma_chains1<GS>(acc, a1, b1);
        } else if constexpr (Ge::MPG == 2 && GS == 2) {
          mfma_chains2x2(acc, ca, cb);
        } else {
#pragma unroll
          for (int g = 0; g < GS; ++g) mfma_chain<Ge::MPG>(acc[g], ca[g], cb[g]);
        }
      }
#pragma unroll
      for (int g = 0; g < GS; ++g) {
        // y += s * t + z * SX for the group
        const float sc = h2f(uint16_t(par[g] & 0xFFFFu)), zc = h2f(uint16_t(par[g] >> 16));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          yacc[i] = __builtin_fmaf(sc, acc[g][i], yacc[i]);
          yacc[i] = __builtin_fmaf(zc, ts[g][i], yacc[i]);
        }
        // INT2's 32 groups per block: the scaling stays with its chain (left
        // free, the compiler moved every group's scaling past the last chain
        // and spilled the accumulators)
        if constexpr (KM == 16) asm volatile("" : "+v"(yacc));
      }
    }
    asm volatile("" ::: "memory");  // the next block's writes stay after this block's reads
  }

  // (6) add the W partial tiles in wave order and store y[m][row] for m < M
  __syncthreads();
  static_assert(Ge::B_BYTES + Ge::P_BYTES >= 1024, "a wave's partial tile fits its LDS area");
  *reinterpret_cast<f32x4*>(lds + Ge::X_BYTES + Ge::T_BYTES + wave * (Ge::B_BYTES + Ge::P_BYTES) + lane * 16) =
      yacc;
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

// Launch for 2..8 activation rows when the shape fits (else returns false and
// the dot-product GEMV serves the call), with W waves per workgroup.
template <int S, int G, int MT, int W, int NBLK>
hipError_t launch_mfma_t(const uq_layout* L, const void* codes, const void* params, const uint16_t* x, float* y,
                         int m, hipStream_t stream) {
  using Ge = MfGeo<S, G, MT, W, NBLK>;
  if constexpr (!Ge::ok) {
    return hipErrorInvalidValue;  // never chosen: mfma_fits() rules the shape out
  } else {
  const int n = int(L->n), k = int(L->k);
  const int64_t blocks = (int64_t(n) + 15) / 16;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const uint8_t* c8 = static_cast<const uint8_t*>(codes);
  const uint8_t* p8 = static_cast<const uint8_t*>(params);
  int nn = n, kk = k, mm = m;
  void* args[] = {&c8, &p8, (void*)&x, &y, &nn, &kk, &mm};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemv_mfma_kernel<S, G, MT, W, NBLK>), dim3(unsigned(blocks)),
                         dim3(64 * W), args, size_t(Ge::LDS), stream);
  }
}

// Blocks per wave, rounded up to 1, 2, 4 or 8 (the block loop is unrolled); 0 past 8.
inline int mfma_nblk(int64_t rowb, int w) {
  const int64_t nb = (rowb + w * kMfBlock - 1) / (w * kMfBlock);
  return nb <= 1 ? 1 : nb <= 2 ? 2 : nb <= 4 ? 4 : nb <= 8 ? 8 : 0;
}

// Whether the shape runs on the matrix-core GEMV: the staged activations fit,
// whole 16-byte parameter slots per row and per wave.
template <int S, int G>
bool mfma_fits(int64_t k, int mt, int w) {
  constexpr int bits = Fmt<S>::bits;
  const int nb = mfma_nblk(k * bits / 8, w);
  if (!nb) return false;
  const int64_t kp = int64_t(nb) * w * kMfBlock * 8 / bits;
  const int64_t qp = kp / w / G * 4;
  return mfma_gemv_scheme<S, G>() && int64_t(mt) * kp * 2 <= kMfXBytes && (k / G) % 4 == 0 && qp % 16 == 0 &&
         (kp / w) % G == 0 && G % Mf<S>::KM == 0;
}

template <int S, int G, int MT, int W>
hipError_t launch_mfma_w(const uq_layout* L, const void* codes, const void* params, const uint16_t* x, float* y,
                         int m, hipStream_t stream) {
  switch (mfma_nblk(L->k * Fmt<S>::bits / 8, W)) {
    case 1: return launch_mfma_t<S, G, MT, W, 1>(L, codes, params, x, y, m, stream);
    case 2: return launch_mfma_t<S, G, MT, W, 2>(L, codes, params, x, y, m, stream);
    case 4: return launch_mfma_t<S, G, MT, W, 4>(L, codes, params, x, y, m, stream);
    case 8: return launch_mfma_t<S, G, MT, W, 8>(L, codes, params, x, y, m, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int S, int G, int W>
hipError_t launch_mfma_m(const uq_layout* L, const void* codes, const void* params, const uint16_t* x, float* y,
                         int m, int mt, hipStream_t stream) {
  if (mt == 2) return launch_mfma_w<S, G, 2, W>(L, codes, params, x, y, m, stream);
  if (mt == 4) return launch_mfma_w<S, G, 4, W>(L, codes, params, x, y, m, stream);
  return launch_mfma_w<S, G, 8, W>(L, codes, params, x, y, m, stream);
}

// The GEMV for INT2 / INT4 / INT8: 2..8 activation rows on the matrix cores
// when the scheme and shape fit, otherwise (and for one row) the dot-product
// kernel.  Eight waves per workgroup, each taking an eighth of every row
// (less work per wave after its loads land; measured on MI355X, INT4 G64
// N11008: M=2 / 4 / 8 8.7 / 9.6 / 14.4 us against 9.3 / 10.7 / 19.1 us on
// four waves).
template <int S, int G>
hipError_t launch_gemv_sel(const uq_layout* L, const void* codes, const void* params, const uint16_t* x, float* y,
                           int m, hipStream_t stream) {
  if constexpr (mfma_gemv_scheme<S, G>()) {
    // With one MFMA and its scaling per group (INT2 G16, INT4 G32) the
    // matrix cores pay off only with more rows (measured on MI355X against
    // the dot product): INT2 G16 N4096 M=8 9.6 -> 8.7 us, but M=2 / 3 / 4
    // 4.6 / 5.7 / 5.7 -> 8.2 / 8.5 / 8.6 us; INT4 G32 N11008 M=3 / 4 / 5 / 8
    // 11.7 / 11.9 / 20.4 / 21.6 -> 11.0 / 11.3 / 16.4 / 16.4 us and N4096
    // M=5 / 8 10.2 / 10.2 -> 6.6 / 6.6 us, but N11008 M=2 8.2 -> 10.1 us and
    // N4096 M=3 / 4 5.6 / 5.7 -> 6.3 / 6.3 us.
    const int min_rows = S == UQ_INT2 ? 5 : S == UQ_INT4 && G == 32 ? (L->n >= 8192 ? 3 : 5) : 2;
    if (m >= min_rows) {
      const int mt = m <= 2 ? 2 : m <= 4 ? 4 : 8;
      if (mfma_fits<S, G>(L->k, mt, 8)) return launch_mfma_m<S, G, 8>(L, codes, params, x, y, m, mt, stream);
    }
  }
  return launch_m<S, G>(L, codes, params, x, y, m, stream);
}

}  // namespace
}  // namespace uq
