// Fused group-wise dequant + GEMV for decode, M <= 8 activation rows
// ("Ultra LLM Engine", Core Components > Fused Kernels: dequantized-weight
// GEMV during single-token decode).
//
// Work split (gfx950, wave64):
//   * A workgroup is 4 waves.  Each wave owns R consecutive weight rows for
//     the whole K range; its 64 lanes split each row into 16-byte code
//     chunks (lane l takes chunks l, l+64, ...), so every 128-bit load
//     instruction of a wave reads 1 KB of one row contiguously from HBM.
//   * Per K block, each lane first issues the loads of the activations it
//     stages, then every weight-chunk load it will need (U chunks x R rows,
//     plus their group parameters), so the block's HBM traffic is in
//     flight while the activations are paired, pre-scaled and written to
//     LDS.  Only then the workgroup synchronises and computes.
//   * The activations sit in LDS paired for the unpacked code layout (see
//     device_common.hpp), unscaled, with two sums per group part: SX = sum x
//     and C = sum B*x, B the fp16 base each code position unpacks with.  The
//     lane forms t = sum (B + q) * x - C = sum q*x with packed fp16 dot
//     products (exact products, fp32 accumulation) and adds s*t + z*SX,
//     which is sum x*(q*s + z).  NF4: a * sum (H[q] + L[q])*x, the codebook
//     split into fp16 high and low parts (two dot products, no rounding of
//     the codebook in the products).
//   * Lane partials are summed across the wave with DPP and lane swizzles.
#pragma once

#include "device_common.hpp"

namespace uq {
namespace {

constexpr int kThreads = 256;
constexpr int kComputeUnits = 256;  // MI355X
constexpr int kWaves = kThreads / 64;
// Activations staged per LDS block (all rows of x together).  INT2 takes
// twice as many: with 5-8 activation rows its K = 4096 then fits one block
// and the loop-free path (INT2 G16 N4096 M=8 15.0 -> 10.6 us); INT8 is
// slower that way (11.3 -> 12.3 us at M=8: 388 VGPRs, one wave per SIMD).
template <int S>
constexpr int x_block() { return S == UQ_INT2 ? 32768 : 16384; }
constexpr int kMaxIPT = 8;  // activation group parts staged per thread and K block, at most

template <int S, int G, int MT = 1>
struct Geo {
  using F = Fmt<S>;
  static constexpr int CW = F::CW, WPD = F::WPD, PPD = F::PPD;
  static constexpr int GP = G < CW ? G : CW;  // codes per group part
  static constexpr int PPC = CW / GP;         // group parts per chunk
  static constexpr int DPG = GP / WPD;        // dwords per group part
  static constexpr int XV = GP / 8;           // 128-bit activation loads per part
  // chunks per lane per group: up to 4096 codes of K, but no more than one
  // LDS block of activations holds
  static constexpr int U0 = (x_block<S>() / MT) / (64 * CW);
  static constexpr int U = U0 < 1 ? 1 : (U0 < 64 / CW ? U0 : 64 / CW);
  static constexpr bool NF = (S == UQ_NF4);
};

template <int S, int G, int R>
struct ChunkRegs {
  uint4 code[R];
  uint32_t par[R][Geo<S, G>::PPC];  // INT: (s | z << 16) per part; NF4: absmax bits
};

// Load 16-byte code chunk `chunk` of each of the wave's R rows, and the
// parameters of the groups it touches.  cbase/pbase point at the wave's first
// row and roff/poff are the (clamped) row offsets -- all wave-uniform -- so
// only the chunk offset is per lane.
template <int S, int G, int R>
__device__ __forceinline__ void load_codes(ChunkRegs<S, G, R>& cr, const uint8_t* __restrict__ cbase,
                                           const int64_t (&roff)[R], int chunk) {
#pragma unroll
  for (int r = 0; r < R; ++r) cr.code[r] = load_stream<uint4>(cbase + roff[r] + uint32_t(chunk) * 16u);
}

template <int S, int G, int R>
__device__ __forceinline__ void load_params(ChunkRegs<S, G, R>& cr, const uint8_t* __restrict__ pbase,
                                            const int64_t (&poff)[R], int chunk) {
  using Gm = Geo<S, G>;
  constexpr int PB = Gm::NF ? 2 : 4;  // bytes of one group's parameters
  const uint32_t gb = uint32_t(chunk) * Gm::CW / G * PB;  // first group of the chunk, in bytes
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint8_t* p = pbase + poff[r] + gb;
    if constexpr (Gm::NF) {
      cr.par[r][0] = load_stream<uint16_t>(p);
    } else if constexpr (Gm::PPC == 1) {
      cr.par[r][0] = load_stream<uint32_t>(p);
    } else if constexpr (Gm::PPC == 2) {
      const uint2 v = load_stream<uint2>(p);
      cr.par[r][0] = v.x;
      cr.par[r][1] = v.y;
    } else {
      const uint4 v = load_stream<uint4>(p);
      cr.par[r][0] = v.x;
      cr.par[r][1] = v.y;
      cr.par[r][2] = v.z;
      cr.par[r][3] = v.w;
    }
  }
}

template <int S, int G, int R>
__device__ __forceinline__ void load_chunk(ChunkRegs<S, G, R>& cr, const uint8_t* __restrict__ cbase,
                                           const uint8_t* __restrict__ pbase, const int64_t (&roff)[R],
                                           const int64_t (&poff)[R], int chunk) {
  load_codes<S, G, R>(cr, cbase, roff, chunk);
  load_params<S, G, R>(cr, pbase, poff, chunk);
}

// Order of a K block's first weight loads: INT4 and NF4 ask for every
// chunk's parameters before the codes (the parameters are needed first and
// are a small share of the bytes; measured on MI355X: INT4 G64 K4096 N11008
// M=1 6.72 -> 6.55 us, G128 6.72 -> 6.42 us, NF4 N14336 10.68 -> 10.42 us);
// INT8 and INT2 load them per chunk after its codes (5.03 vs 5.12 us, 3.99
// vs 4.05 us the other way).
template <int S>
constexpr bool params_first() { return S == UQ_INT4 || S == UQ_NF4; }

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ _Float16 half_of(const uint4& v, int e) {
  const uint32_t d = dword_of(v, e >> 1);
  return __builtin_bit_cast(_Float16, uint16_t((e & 1) ? (d >> 16) : (d & 0xFFFFu)));
}

template <int PPD>
__device__ __forceinline__ void load_pairs(const uint32_t* src, f16x2 (&xp)[PPD]) {
  if constexpr (PPD >= 4) {
#pragma unroll
    for (int q = 0; q < PPD / 4; ++q) {
      const uint4 v = reinterpret_cast<const uint4*>(src)[q];
      xp[4 * q] = as_h2(v.x);
      xp[4 * q + 1] = as_h2(v.y);
      xp[4 * q + 2] = as_h2(v.z);
      xp[4 * q + 3] = as_h2(v.w);
    }
  } else {
    const uint2 v = reinterpret_cast<const uint2*>(src)[0];
    xp[0] = as_h2(v.x);
    xp[1] = as_h2(v.y);
  }
}

template <int S>
__device__ __forceinline__ void unpack_dword(uint32_t w, f16x2 (&hp)[Fmt<S>::PPD]) {
  unpack_pairs<S>(w, hp);
}

// NF4: byte j of w -> the high and low fp16 parts of its two codes' values
// (one 8-byte table entry: high pair, low pair).
__device__ __forceinline__ void unpack_nf4(uint32_t w, const uint2* lut, f16x2 (&hp)[4], f16x2 (&lp)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint2 e = lut[(w >> (8 * j)) & 0xFFu];
    hp[j] = as_h2(e.x);
    lp[j] = as_h2(e.y);
  }
}

// y += s * t + z * SX for one group part (t = the accumulator, which started
// at -C); NF4: y += a * t.
template <bool NF, int MT, int PPC>
__device__ __forceinline__ void apply_group(uint32_t par, const float (&acc)[MT], const float2 (&cv)[MT][PPC],
                                            int pp, float (&acc_y)[MT]) {
  if constexpr (NF) {
    const float a = h2f(uint16_t(par));
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) acc_y[mm] = __builtin_fmaf(a, acc[mm], acc_y[mm]);
  } else {
    const float s = h2f(uint16_t(par & 0xFFFFu));
    const float z = h2f(uint16_t(par >> 16));
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
      acc_y[mm] = __builtin_fmaf(s, acc[mm], acc_y[mm]);
      acc_y[mm] = __builtin_fmaf(z, cv[mm][pp].y, acc_y[mm]);
    }
  }
}

// ONE: the whole K range fits one LDS block of activations and one group of
// 64*U chunks per lane, so the kernel body is loop-free.  (With a loop, the
// compiler must assume loads from the previous trip may still be landing in
// the registers it is about to reuse, and it waits for them at the loop head,
// which stalls the first trip's weight loads behind the activation loads.)
template <int S, int G, int MT, int R, bool ONE, int IPT>
__global__ __launch_bounds__(kThreads) void gemv_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ params,
    const uint16_t* __restrict__ x, float* __restrict__ y, int n, int k, int m,
    int kb_max) {
  using Gm = Geo<S, G, MT>;
  constexpr int CW = Gm::CW, WPD = Gm::WPD, PPD = Gm::PPD, GP = Gm::GP;
  constexpr int PPC = Gm::PPC, DPG = Gm::DPG, XV = Gm::XV, U = Gm::U;
  constexpr bool NF = Gm::NF;
  // Each thread stages IPT activation group parts per K block (IPT * 256
  // covers the block; chosen at launch).
  constexpr int kIPT = IPT;

  extern __shared__ uint4 lds4[];
  uint32_t* lds = reinterpret_cast<uint32_t*>(lds4);
  uint2* lut = reinterpret_cast<uint2*>(lds);       // NF4: 256 x (high pair, low pair)
  uint32_t* xs = lds + (NF ? 512 : 0);              // [MT][kb_max/2] fp16 pairs
  float2* cs = reinterpret_cast<float2*>(xs + MT * (kb_max / 2));  // [MT][kb_max/GP]: (-C, SX)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int64_t row0 = (int64_t(blockIdx.x) * kWaves + wave) * R;
  const size_t rowb = size_t(k) * Fmt<S>::bits / 8;
  const int ng = k / G;
  // Wave-uniform addressing: base pointers at the wave's first row, clamped
  // row offsets (rows past n re-read row n-1 and are not stored).
  const uint8_t* cbase = codes + size_t(row0) * rowb;
  const uint8_t* pbase = params + size_t(row0) * size_t(ng) * (NF ? 2 : 4);
  int64_t roff[R], poff[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t rr = row0 + r < n ? r : int64_t(n) - 1 - row0;
    roff[r] = rr * int64_t(rowb);
    poff[r] = rr * int64_t(ng) * (NF ? 2 : 4);
  }

  if constexpr (NF) {
    static_assert(kThreads == 256, "the NF4 byte table takes one entry per thread");
    // byte b -> the codes' values C[b & 15], C[b >> 4] as a pair of fp16 high
    // parts h = fp16(C) and a pair of low parts l = fp16(C - h): h + l holds
    // C to about 2^-22, and the dot products of x with h and with l are exact
    // in fp32, so the NF4 products carry no rounding of the codebook.
    const float c0 = nf4_value(tid & 15), c1 = nf4_value(tid >> 4);
    const _Float16 h0 = _Float16(c0), h1 = _Float16(c1);
    lut[tid] = make_uint2(as_u32(f16x2{h0, h1}), as_u32(f16x2{_Float16(c0 - float(h0)), _Float16(c1 - float(h1))}));
  }

  float acc_y[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) acc_y[r][mm] = 0.0f;

  // One K block: stage its activations, stream its weight chunks, accumulate.
  auto k_block = [&](const int kb0) __attribute__((always_inline)) {
    const int kb = ONE ? k : (k - kb0 < kb_max ? k - kb0 : kb_max);
    const int nch = kb / CW;
    const int64_t ch0 = kb0 / CW;
    const int n_items = MT * nch * PPC;

    // (1) activation loads for the parts this thread stages (L2 hits; issued
    //     first so they return first)
    //     Loads are never predicated: out-of-range items and chunks load a
    //     clamped, valid address and are ignored later.  (Conditionally issued
    //     loads leave the compiler unsure how many loads follow a given one,
    //     and it then waits for all of them.)
    uint4 xr[kIPT][XV];
#pragma unroll
    for (int s = 0; s < kIPT; ++s) {
      const int it0 = tid + s * kThreads;
      const int it = it0 < n_items ? it0 : n_items - 1;
      const int mm = it / (nch * PPC);
      const int rem = it - mm * (nch * PPC);
      const int c = rem / PPC, pp = rem - c * PPC;
      const uint4* src = reinterpret_cast<const uint4*>(
          x + size_t(mm < m ? mm : 0) * size_t(k) + kb0 + c * CW + pp * GP);
#pragma unroll
      for (int v = 0; v < XV; ++v) xr[s][v] = src[v];
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the activation loads ahead of the weight loads
    // (2) every weight chunk of the first 64*U columns, for all R rows
    ChunkRegs<S, G, R> cur[U];
    if constexpr (params_first<S>()) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = lane + 64 * u;
        load_params<S, G, R>(cur[u], pbase, poff, int(ch0) + (c < nch ? c : nch - 1));
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = lane + 64 * u;
        load_codes<S, G, R>(cur[u], cbase, roff, int(ch0) + (c < nch ? c : nch - 1));
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = lane + 64 * u;
        load_chunk<S, G, R>(cur[u], cbase, pbase, roff, poff, int(ch0) + (c < nch ? c : nch - 1));
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // and all weight loads ahead of the staging work

    // (3) stage: pair, sum; write LDS
    __syncthreads();  // LDS free (previous K block done)
    // Threads past the last item redo the last one (same values, same LDS
    // words), so the staging has no branch for the loads to sink into.
#pragma unroll
    for (int s = 0; s < kIPT; ++s) {
      {
        const int it0 = tid + s * kThreads;
        const int it = it0 < n_items ? it0 : n_items - 1;
        const int mm = it / (nch * PPC);
        const int rem = it - mm * (nch * PPC);
        const int c = rem / PPC, pp = rem - c * PPC;
        const bool live = mm < m;
        const f16x2 one2 = {_Float16(1.0f), _Float16(1.0f)};
        float sx = 0.0f, sxb = 0.0f;  // sum x, sum B*x
#pragma unroll
        for (int dl = 0; dl < DPG; ++dl) {
          const int dd = pp * DPG + dl;
          uint32_t d[WPD / 2];  // this code dword's activations, natural fp16 pairs
#pragma unroll
          for (int j = 0; j < WPD / 2; ++j) d[j] = live ? dword_of(xr[s][(dl * WPD / 2 + j) >> 2], (dl * WPD / 2 + j) & 3) : 0u;
          f16x2 pr[PPD];
          pair_activations<S>(d, pr);
          if constexpr (!NF) {
#pragma unroll
            for (int j = 0; j < WPD / 2; ++j) sx = __builtin_amdgcn_fdot2(as_h2(d[j]), one2, sx, false);
#pragma unroll
            for (int j = 0; j < PPD; ++j) {
              const _Float16 b = _Float16(Slot<S>::base(j));  // a power of two: exact products
              sxb = __builtin_amdgcn_fdot2(pr[j], f16x2{b, b}, sxb, false);
            }
          }
          uint32_t* dst = xs + mm * (kb_max / 2) + (dd * nch + c) * PPD;
          if constexpr (PPD == 8) {
            reinterpret_cast<uint4*>(dst)[0] = make_uint4(as_u32(pr[0]), as_u32(pr[1]), as_u32(pr[2]), as_u32(pr[3]));
            reinterpret_cast<uint4*>(dst)[1] = make_uint4(as_u32(pr[4]), as_u32(pr[5]), as_u32(pr[6]), as_u32(pr[7]));
          } else if constexpr (PPD == 4) {
            reinterpret_cast<uint4*>(dst)[0] = make_uint4(as_u32(pr[0]), as_u32(pr[1]), as_u32(pr[2]), as_u32(pr[3]));
          } else {
            reinterpret_cast<uint2*>(dst)[0] = make_uint2(as_u32(pr[0]), as_u32(pr[1]));
          }
        }
        if constexpr (!NF) cs[mm * (kb_max / GP) + pp * nch + c] = make_float2(-sxb, sx);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // no weight-dependent math above the barrier
    __syncthreads();

    // (4) compute; K blocks wider than 64*U chunks load each further group
    //     just before using it (many waves per SIMD cover that latency)
    // one group of 64*U chunks per lane; further groups (long K) reload `cur`
    auto chunk_group = [&](const int cg) __attribute__((always_inline)) {
      if (cg > 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = cg + lane + 64 * u;
          load_chunk<S, G, R>(cur[u], cbase, pbase, roff, poff, int(ch0) + (c < nch ? c : nch - 1));
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // One chunk at a time: keep the scheduler from interleaving chunks,
        // which would hold every chunk's temporaries live at once.
        __builtin_amdgcn_sched_barrier(0);
        // No branch around the math either (it would invite the compiler to
        // sink the weight loads into it): a lane past the last chunk works
        // on its clamped chunk and adds it with scale and zero set to 0.
        const int c0 = cg + lane + 64 * u;
        const bool valid = c0 < nch;
        const int c = valid ? c0 : nch - 1;
        if constexpr (MT <= 2) {
          // Row-inner: the chunk's activation pairs stay in registers and each
          // row's math waits only for that row's own load.
          f16x2 xp[MT][4][PPD];
#pragma unroll
          for (int mm = 0; mm < MT; ++mm)
#pragma unroll
            for (int dd = 0; dd < 4; ++dd) load_pairs<PPD>(xs + mm * (kb_max / 2) + (dd * nch + c) * PPD, xp[mm][dd]);
          float2 cv[MT][PPC];
          if constexpr (!NF) {
#pragma unroll
            for (int mm = 0; mm < MT; ++mm)
#pragma unroll
              for (int pp = 0; pp < PPC; ++pp) cv[mm][pp] = cs[mm * (kb_max / GP) + pp * nch + c];
          }
#pragma unroll
          for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int pp = 0; pp < PPC; ++pp) {
              float acc[MT];
#pragma unroll
              for (int mm = 0; mm < MT; ++mm) acc[mm] = NF ? 0.0f : cv[mm][pp].x;  // starts at -C
#pragma unroll
              for (int dl = 0; dl < DPG; ++dl) {
                const int dd = pp * DPG + dl;
                f16x2 hp[PPD], lp[NF ? PPD : 1];
                if constexpr (NF) unpack_nf4(dword_of(cur[u].code[r], dd), lut, hp, lp);
                else unpack_dword<S>(dword_of(cur[u].code[r], dd), hp);
                // (the same order of additions as the dword-outer path below)
#pragma unroll
                for (int mm = 0; mm < MT; ++mm)
#pragma unroll
                  for (int j = 0; j < PPD; ++j) {
                    acc[mm] = __builtin_amdgcn_fdot2(hp[j], xp[mm][dd][j], acc[mm], false);
                    if constexpr (NF) acc[mm] = __builtin_amdgcn_fdot2(lp[j], xp[mm][dd][j], acc[mm], false);
                  }
              }
              apply_group<NF>(valid ? cur[u].par[r][pp] : 0u, acc, cv, pp, acc_y[r]);
            }
          }
        } else {
          // Dword-outer: each activation pair read from LDS serves all R rows.
#pragma unroll
          for (int pp = 0; pp < PPC; ++pp) {
            float2 cv[MT][PPC];
            if constexpr (!NF) {
#pragma unroll
              for (int mm = 0; mm < MT; ++mm) cv[mm][pp] = cs[mm * (kb_max / GP) + pp * nch + c];
            }
            float acc[R][MT];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
              for (int mm = 0; mm < MT; ++mm) acc[r][mm] = NF ? 0.0f : cv[mm][pp].x;  // starts at -C
#pragma unroll
            for (int dl = 0; dl < DPG; ++dl) {
              const int dd = pp * DPG + dl;
              f16x2 hp[R][PPD];
              f16x2 lp[R][NF ? 4 : 1];
#pragma unroll
              for (int r = 0; r < R; ++r) {
                if constexpr (NF) unpack_nf4(dword_of(cur[u].code[r], dd), lut, hp[r], lp[r]);
                else unpack_dword<S>(dword_of(cur[u].code[r], dd), hp[r]);
              }
#pragma unroll
              for (int mm = 0; mm < MT; ++mm) {
                f16x2 xq[PPD];
                load_pairs<PPD>(xs + mm * (kb_max / 2) + (dd * nch + c) * PPD, xq);
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                  for (int j = 0; j < PPD; ++j) {
                    acc[r][mm] = __builtin_amdgcn_fdot2(hp[r][j], xq[j], acc[r][mm], false);
                    if constexpr (NF) acc[r][mm] = __builtin_amdgcn_fdot2(lp[r][j], xq[j], acc[r][mm], false);
                  }
              }
            }
#pragma unroll
            for (int r = 0; r < R; ++r) apply_group<NF>(valid ? cur[u].par[r][pp] : 0u, acc[r], cv, pp, acc_y[r]);
          }
        }
      }
    };
    if constexpr (ONE) {
      chunk_group(0);
    } else {
      for (int cg = 0; cg < nch; cg += 64 * U) chunk_group(cg);
    }
  };
  if constexpr (ONE) {
    k_block(0);
  } else {
    for (int kb0 = 0; kb0 < k; kb0 += kb_max) k_block(kb0);
  }

  // Reduce lane partials and store: four (row, m) outputs per swap-reduction,
  // a last group of fewer padded with zeros.  Each output's additions do not
  // depend on the other three, so every (row, m) is summed in one order
  // whatever R and MT are.
  constexpr int NV = R * MT;
  float* yv = &acc_y[0][0];
#pragma unroll
  for (int q = 0; q < NV; q += 4) {
    const float v = wave_sum4(yv[q], q + 1 < NV ? yv[q + 1] : 0.0f, q + 2 < NV ? yv[q + 2] : 0.0f,
                              q + 3 < NV ? yv[q + 3] : 0.0f);
    const int slot = q + ((lane >> 4) == 1 ? 2 : (lane >> 4) == 2 ? 1 : (lane >> 4));  // a, c, b, d
    const int r = slot / MT, mm = slot - r * MT;
    if ((lane & 15) == 0 && slot < NV && row0 + r < n && mm < m) y[size_t(mm) * size_t(n) + size_t(row0 + r)] = v;
  }
}

// Weight rows per wave.  Four for a single activation row (two for INT8,
// whose rows hold twice the bytes: N4096 M=1 5.43 -> 5.03 us; INT4 is slower
// with two, 6.79 -> 7.24 us, and every scheme with eight; two for NF4, the
// fastest of one to five rows or within 3 % of it at every shape tried:
// K4096 N14336 9.79 -> 9.18 us, N11008 8.18 -> 8.07, N4096 5.03 -> 4.75,
// K14336 N4096 16.2 -> 11.4); with two or more activation rows the
// per-row state grows and two rows per wave keep more waves resident
// (measured on MI355X: 5-14 % faster for INT4 M=4 and INT8 M=8).  INT2 keeps
// four (its LDS traffic per code byte is the highest).
template <int S, int MT>
constexpr int rows_per_wave() {
  if (MT == 1) return S == UQ_INT8 || S == UQ_NF4 ? 2 : 4;
  return S == UQ_INT2 ? 4 : 2;
}

template <int S, int G, int MT, int R, bool ONE>
hipError_t launch_ipt(int ipt, dim3 grid, void** args, size_t shmem, hipStream_t stream) {
  const void* fn = ipt == 1   ? reinterpret_cast<const void*>(&gemv_kernel<S, G, MT, R, ONE, 1>)
                   : ipt == 2 ? reinterpret_cast<const void*>(&gemv_kernel<S, G, MT, R, ONE, 2>)
                   : ipt == 4 ? reinterpret_cast<const void*>(&gemv_kernel<S, G, MT, R, ONE, 4>)
                              : reinterpret_cast<const void*>(&gemv_kernel<S, G, MT, R, ONE, 8>);
  return hipLaunchKernel(fn, grid, dim3(kThreads), args, shmem, stream);
}

// Activations staged per K block: one LDS block of x, at most kMaxIPT group
// parts per thread (kMaxIPT * kThreads parts of GP activations across the MT
// rows), at most K.
template <int S, int G, int MT>
int block_k(int k) {
  using Gm = Geo<S, G, MT>;
  int kb_max = x_block<S>() / MT;
  if (kb_max > k) kb_max = k;
  if (int64_t(MT) * (kb_max / Gm::GP) > int64_t(kMaxIPT) * kThreads) kb_max = kMaxIPT * kThreads * Gm::GP / MT;
  return kb_max;
}

// Whether the whole K range is one K block and one group of 64 * U chunks per
// lane: the loop-free kernel body.
template <int S, int G, int MT>
bool one_block(int k) {
  using Gm = Geo<S, G, MT>;
  return block_k<S, G, MT>(k) == k && k <= 64 * Gm::U * Gm::CW;
}

template <int S, int G, int MT, int R>
hipError_t launch(const uq_layout* L, const void* codes, const void* params, const uint16_t* x,
                  float* y, int m, hipStream_t stream) {
  using Gm = Geo<S, G, MT>;
  const int k = int(L->k), n = int(L->n);
  int kb_max = block_k<S, G, MT>(k);
  const size_t shmem = (Gm::NF ? 2048 : 0) + size_t(MT) * kb_max * 2 + (Gm::NF ? 0 : size_t(MT) * (kb_max / Gm::GP) * 8);
  const int64_t rows_per_block = kWaves * R;
  const int64_t blocks = (int64_t(n) + rows_per_block - 1) / rows_per_block;  // n < 2^31: no overflow in int64
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid{unsigned(blocks)};
  const uint8_t* c8 = static_cast<const uint8_t*>(codes);
  const uint8_t* p8 = static_cast<const uint8_t*>(params);
  void* args[] = {&c8, &p8, (void*)&x, &y, (void*)&n, (void*)&k, &m, &kb_max};
  const int items = MT * (kb_max / Gm::GP);  // staged activation parts per K block
  const int ipt = items <= kThreads ? 1 : items <= 2 * kThreads ? 2 : items <= 4 * kThreads ? 4 : 8;
  const bool one = one_block<S, G, MT>(k);
  return one ? launch_ipt<S, G, MT, R, true>(ipt, grid, args, shmem, stream)
             : launch_ipt<S, G, MT, R, false>(ipt, grid, args, shmem, stream);
}

template <int S, int G>
hipError_t launch_m(const uq_layout* L, const void* codes, const void* params, const uint16_t* x,
                    float* y, int m, hipStream_t stream) {
  if (m == 1) {
    // A weight matrix with too few rows to give every compute unit a
    // workgroup at the usual rows per wave takes one row per wave, four times
    // the workgroups (measured on MI355X, INT4 G32 K256 N768: 2.98 us with
    // four rows per wave, 2.65 with two, 2.46 with one).
    constexpr int R = rows_per_wave<S, 1>();
    if ((L->n + int64_t(kWaves) * R - 1) / (int64_t(kWaves) * R) < kComputeUnits)
      return launch<S, G, 1, 1>(L, codes, params, x, y, m, stream);
    // Past one K block (the kernel loops over K blocks and chunk groups) two
    // rows per wave beat four (measured on MI355X, M=1: INT4 G64 K14336 N4096
    // 11.4 -> 8.7 us, K11008 N4096 9.7 -> 7.7, K8192 N8192 10.2 -> 8.9, INT2
    // G16 K14336 N4096 11.0 -> 8.8; one row per wave slower than two at every
    // such shape), while four stay faster within one block (K4096 N11008 6.53
    // against 6.75 us).
    if constexpr (R > 2) {
      if (!one_block<S, G, 1>(int(L->k))) return launch<S, G, 1, 2>(L, codes, params, x, y, m, stream);
    }
    return launch<S, G, 1, R>(L, codes, params, x, y, m, stream);
  }
  if (m == 2) return launch<S, G, 2, rows_per_wave<S, 2>()>(L, codes, params, x, y, m, stream);
  if (m <= 4) return launch<S, G, 4, rows_per_wave<S, 4>()>(L, codes, params, x, y, m, stream);
  return launch<S, G, 8, rows_per_wave<S, 8>()>(L, codes, params, x, y, m, stream);
}

}  // namespace
}  // namespace uq
