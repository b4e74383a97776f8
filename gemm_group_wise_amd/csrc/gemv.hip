// Fused group-wise dequant + GEMV for decode, M <= 8 activation rows
// ("Ultra LLM Engine", Core Components > Fused Kernels: dequantized-weight
// GEMV during single-token decode).
//
// Work split (gfx950, wave64):
//   * A workgroup is 4 waves.  Each wave owns R consecutive weight rows for
//     the whole K range; its 64 lanes split each row into 16-byte code
//     chunks (lane l takes chunks l, l+64, ...), so every 128-bit load
//     instruction of a wave reads 1 KB of one row contiguously from HBM.
//   * The activations are staged once per workgroup in LDS, already paired
//     and pre-scaled for the unpacked code layout (see device_common.hpp),
//     together with two per-group-part sums: SX = sum x and
//     C = 1024 * sum x'.  K is walked in LDS-sized blocks.
//   * Per group part the lane forms t = sum (1024 + cls*q) * x/cls - C
//     = sum q*x with packed fp16 dot products (fp32 accumulation), then
//     y += s*t + z*SX, which is sum x*(q*s + z) (NF4: y += a * sum C[q]*x).
//   * Lane partials are summed across the wave with DPP and lane swizzles.
#include "device_common.hpp"

namespace uq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

template <int S, int G>
struct Geo {
  using F = Fmt<S>;
  static constexpr int CW = F::CW, WPD = F::WPD, PPD = F::PPD;
  static constexpr int GP = G < CW ? G : CW;  // codes per group part
  static constexpr int PPC = CW / GP;         // group parts per chunk
  static constexpr int DPG = GP / WPD;        // dwords per group part
  static constexpr bool NF = (S == UQ_NF4);
};

// Load the 16-byte code chunk `c` (absolute chunk index) of each of the R
// rows, plus the parameters of the groups it touches.
template <int S, int G, int R>
struct ChunkRegs {
  uint4 code[R];
  uint32_t par[R][Geo<S, G>::PPC];  // INT: (s | z << 16) per part; NF4: absmax bits
};

template <int S, int G, int R>
__device__ __forceinline__ void load_chunk(ChunkRegs<S, G, R>& cr, const uint8_t* __restrict__ codes,
                                           const uint8_t* __restrict__ params, const int (&rows)[R],
                                           size_t rowb, int ng, int64_t chunk) {
  using Gm = Geo<S, G>;
#pragma unroll
  for (int r = 0; r < R; ++r)
    cr.code[r] = *reinterpret_cast<const uint4*>(codes + size_t(rows[r]) * rowb + size_t(chunk) * 16);
  const int64_t g0 = chunk * Gm::CW / G;  // first group of the chunk
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t gi = int64_t(rows[r]) * ng + g0;
    if constexpr (Gm::NF) {
      cr.par[r][0] = *reinterpret_cast<const uint16_t*>(params + gi * 2);
    } else if constexpr (Gm::PPC == 1) {
      cr.par[r][0] = *reinterpret_cast<const uint32_t*>(params + gi * 4);
    } else if constexpr (Gm::PPC == 2) {
      const uint2 v = *reinterpret_cast<const uint2*>(params + gi * 4);
      cr.par[r][0] = v.x;
      cr.par[r][1] = v.y;
    } else {
      const uint4 v = *reinterpret_cast<const uint4*>(params + gi * 4);
      cr.par[r][0] = v.x;
      cr.par[r][1] = v.y;
      cr.par[r][2] = v.z;
      cr.par[r][3] = v.w;
    }
  }
}

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

template <int S, int G, int MT, int R>
__global__ __launch_bounds__(kThreads) void gemv_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ params,
    const uint16_t* __restrict__ x, float* __restrict__ y, int n, int k, int m,
    int kb_max) {
  using Gm = Geo<S, G>;
  using SL = Slot<S>;
  constexpr int CW = Gm::CW, WPD = Gm::WPD, PPD = Gm::PPD, GP = Gm::GP;
  constexpr int PPC = Gm::PPC, DPG = Gm::DPG;
  constexpr bool NF = Gm::NF;

  extern __shared__ uint32_t lds[];
  uint32_t* lut = lds;                              // NF4: 256 fp16 pairs
  uint32_t* xs = lds + (NF ? 256 : 0);              // [MT][kb_max/2] fp16 pairs
  float2* cs = reinterpret_cast<float2*>(xs + MT * (kb_max / 2));  // [MT][kb_max/GP]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row0 = (int64_t(blockIdx.x) * kWaves + wave) * R;
  const size_t rowb = size_t(k) * Fmt<S>::bits / 8;
  const int ng = k / G;
  int rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rows[r] = int(row0 + r < n ? row0 + r : n - 1);

  if constexpr (NF) {
    // byte b -> (fp16(C[b & 15]), fp16(C[b >> 4]))
    const _Float16 lo = _Float16(nf4_value(tid & 15)), hi = _Float16(nf4_value(tid >> 4));
    lut[tid] = as_u32(f16x2{lo, hi});
  }

  float acc_y[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) acc_y[r][mm] = 0.0f;

  for (int kb0 = 0; kb0 < k; kb0 += kb_max) {
    const int kb = k - kb0 < kb_max ? k - kb0 : kb_max;
    const int nch = kb / CW;
    const int64_t ch0 = kb0 / CW;

    // Issue the first chunk's HBM loads before staging, to overlap latency.
    ChunkRegs<S, G, R> cur;
    if (lane < nch) load_chunk<S, G, R>(cur, codes, params, rows, rowb, ng, ch0 + lane);

    __syncthreads();  // LDS free (previous K block done)
    // Stage x for this K block: items (m, chunk, part).
    for (int it = tid; it < MT * nch * PPC; it += kThreads) {
      const int mm = it / (nch * PPC);
      const int rem = it - mm * (nch * PPC);
      const int c = rem / PPC, pp = rem - c * PPC;
      const int kbase = kb0 + c * CW + pp * GP;
      const bool live = mm < m;
      const uint16_t* xr = x + size_t(live ? mm : 0) * size_t(k) + kbase;
      float sx = 0.0f, sxp = 0.0f;
#pragma unroll
      for (int dl = 0; dl < DPG; ++dl) {
        const int dd = pp * DPG + dl;
        _Float16 v[WPD];
#pragma unroll
        for (int q = 0; q < WPD; q += 8) {
          if constexpr (WPD >= 8) {
            const uint4 raw = *reinterpret_cast<const uint4*>(xr + dl * WPD + q);
            const uint16_t* hv = reinterpret_cast<const uint16_t*>(&raw);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[q + e] = live ? __builtin_bit_cast(_Float16, hv[e]) : _Float16(0);
          }
        }
        if constexpr (WPD == 4) {
          const uint2 raw = *reinterpret_cast<const uint2*>(xr + dl * WPD);
          const uint16_t* hv = reinterpret_cast<const uint16_t*>(&raw);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = live ? __builtin_bit_cast(_Float16, hv[e]) : _Float16(0);
        }
        f16x2 pr[PPD];
#pragma unroll
        for (int i = 0; i < WPD; ++i) {
          const float xf = float(v[i]);
          const _Float16 xp = _Float16(xf * SL::inv_cls(i));
          sx += xf;
          sxp += float(xp);
          pr[SL::pair(i)][SL::half(i)] = xp;
        }
        uint32_t* dst = xs + mm * (kb_max / 2) + (dd * nch + c) * PPD;
#pragma unroll
        for (int j = 0; j < PPD; ++j) dst[j] = as_u32(pr[j]);
      }
      if constexpr (!NF) cs[mm * (kb_max / GP) + pp * nch + c] = make_float2(1024.0f * sxp, sx);
    }
    __syncthreads();

    for (int c = lane; c < nch; c += 64) {
      ChunkRegs<S, G, R> nxt;
      if (c + 64 < nch) load_chunk<S, G, R>(nxt, codes, params, rows, rowb, ng, ch0 + c + 64);
#pragma unroll
      for (int pp = 0; pp < PPC; ++pp) {
        float acc[R][MT];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int mm = 0; mm < MT; ++mm) acc[r][mm] = 0.0f;
#pragma unroll
        for (int dl = 0; dl < DPG; ++dl) {
          const int dd = pp * DPG + dl;
          f16x2 hp[R][PPD];
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const uint32_t w = dword_of(cur.code[r], dd);
            if constexpr (NF) {
#pragma unroll
              for (int j = 0; j < 4; ++j) hp[r][j] = as_h2(lut[(w >> (8 * j)) & 0xFFu]);
            } else {
              unpack_pairs<S>(w, hp[r]);
            }
          }
#pragma unroll
          for (int mm = 0; mm < MT; ++mm) {
            const uint32_t* src = xs + mm * (kb_max / 2) + (dd * nch + c) * PPD;
            f16x2 xp[PPD];
#pragma unroll
            for (int j = 0; j < PPD; ++j) xp[j] = as_h2(src[j]);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
              for (int j = 0; j < PPD; ++j)
                acc[r][mm] = __builtin_amdgcn_fdot2(hp[r][j], xp[j], acc[r][mm], false);
          }
        }
        if constexpr (NF) {
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const float a = h2f(uint16_t(cur.par[r][0]));
#pragma unroll
            for (int mm = 0; mm < MT; ++mm) acc_y[r][mm] = __builtin_fmaf(a, acc[r][mm], acc_y[r][mm]);
          }
        } else {
          float2 cv[MT];
#pragma unroll
          for (int mm = 0; mm < MT; ++mm) cv[mm] = cs[mm * (kb_max / GP) + pp * nch + c];
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const float s = h2f(uint16_t(cur.par[r][pp] & 0xFFFFu));
            const float z = h2f(uint16_t(cur.par[r][pp] >> 16));
#pragma unroll
            for (int mm = 0; mm < MT; ++mm) {
              acc_y[r][mm] = __builtin_fmaf(s, acc[r][mm] - cv[mm].x, acc_y[r][mm]);
              acc_y[r][mm] = __builtin_fmaf(z, cv[mm].y, acc_y[r][mm]);
            }
          }
        }
      }
      cur = nxt;
    }
  }

  // Reduce lane partials and store.
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
      const float v = wave_sum(acc_y[r][mm]);
      if (lane == r * MT + mm && row0 + r < n && mm < m) y[size_t(mm) * size_t(n) + size_t(row0 + r)] = v;
    }
}

template <int S, int G, int MT, int R>
hipError_t launch(const uq_layout* L, const void* codes, const void* params, const uint16_t* x,
                  float* y, int m, hipStream_t stream) {
  using Gm = Geo<S, G>;
  const int k = int(L->k), n = int(L->n);
  int kb_max = 16384 / MT;
  if (kb_max > k) kb_max = k;
  const size_t shmem = (Gm::NF ? 1024 : 0) + size_t(MT) * kb_max * 2 +
                       (Gm::NF ? 0 : size_t(MT) * (kb_max / Gm::GP) * 8);
  const int rows_per_block = kWaves * R;
  const dim3 grid(unsigned((n + rows_per_block - 1) / rows_per_block)), block(kThreads);
  const uint8_t* c8 = static_cast<const uint8_t*>(codes);
  const uint8_t* p8 = static_cast<const uint8_t*>(params);
  void* args[] = {&c8, &p8, &x, &y, (void*)&n, (void*)&k, &m, &kb_max};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemv_kernel<S, G, MT, R>), grid, block, args,
                         shmem, stream);
}

template <int S, int G>
hipError_t launch_m(const uq_layout* L, const void* codes, const void* params, const uint16_t* x,
                    float* y, int m, hipStream_t stream) {
  if (m == 1) return launch<S, G, 1, 4>(L, codes, params, x, y, m, stream);
  if (m == 2) return launch<S, G, 2, 4>(L, codes, params, x, y, m, stream);
  if (m <= 4) return launch<S, G, 4, 4>(L, codes, params, x, y, m, stream);
  return launch<S, G, 8, 4>(L, codes, params, x, y, m, stream);
}

}  // namespace

hipError_t launch_gemv(const uq_layout* L, const void* codes, const void* params, const uint16_t* x,
                       float* y, int m, hipStream_t stream) {
  switch (L->scheme * 1000 + L->group) {
    case UQ_INT2 * 1000 + 16: return launch_m<UQ_INT2, 16>(L, codes, params, x, y, m, stream);
    case UQ_INT2 * 1000 + 32: return launch_m<UQ_INT2, 32>(L, codes, params, x, y, m, stream);
    case UQ_INT2 * 1000 + 64: return launch_m<UQ_INT2, 64>(L, codes, params, x, y, m, stream);
    case UQ_INT2 * 1000 + 128: return launch_m<UQ_INT2, 128>(L, codes, params, x, y, m, stream);
    case UQ_INT4 * 1000 + 32: return launch_m<UQ_INT4, 32>(L, codes, params, x, y, m, stream);
    case UQ_INT4 * 1000 + 64: return launch_m<UQ_INT4, 64>(L, codes, params, x, y, m, stream);
    case UQ_INT4 * 1000 + 128: return launch_m<UQ_INT4, 128>(L, codes, params, x, y, m, stream);
    case UQ_INT8 * 1000 + 64: return launch_m<UQ_INT8, 64>(L, codes, params, x, y, m, stream);
    case UQ_INT8 * 1000 + 128: return launch_m<UQ_INT8, 128>(L, codes, params, x, y, m, stream);
    case UQ_NF4 * 1000 + 64: return launch_m<UQ_NF4, 64>(L, codes, params, x, y, m, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace uq
