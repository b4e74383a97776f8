// Activation-quantized GEMV for decode (M <= 8) with INT2/4/8 weights ("Ultra
// LLM Engine", Core Components > Quantized Model: the quantized layers quantize
// their activations on the fly; the scheme is not given there).
//
// The activations are quantized to int8 per (activation row, weight group):
// a = max |x| over the group, codes q = rint(x * (127 / a)) in fp32, clamped to
// +-127, scale s_x = a / 127.  With the INT weights w' = q_w * s + z:
//     y[m][n] = sum_g s_x * (s * D + z * Q),  D = sum q_w * q_x,  Q = sum q_x,
// where D and Q are exact integer sums (v_dot4 on int8 lanes, 4 products per
// instruction) and only the per-group scaling is floating point (fp32).
//
//   * A workgroup is 4 waves; each wave owns 4 weight rows (2 when x has
//     five to eight rows, or one row of INT8 / INT2 weights), so the staged
//     activations serve 16 (8) weight rows.  Per K block the workgroup quantizes every activation row into
//     LDS once: int8 codes laid out in the order the
//     unpacked weight lanes take them (INT4: even codes then odd codes of each
//     8; INT2: crumb j of each byte), the code sum of every 16, and s_x.
//   * Lanes then stream 16-byte chunks of their rows' codes (coalesced along
//     K), unpack them to int8 lanes with masks (INT8 flips the sign bit:
//     q - 128, corrected by 128 * Q), and accumulate D per group portion;
//     each portion is scaled once per (row, activation row).
//   * Lane partials are summed across the wave with lane swaps.
#include "device_common.hpp"

namespace uq {
namespace {

constexpr int kA8Threads = 256;
constexpr int kA8Waves = kA8Threads / 64;
// Weight rows per wave: four, or two for eight activation rows (their
// accumulators and activation codes would otherwise leave room for only one
// wave per SIMD), and two for a single activation row of INT8 or INT2
// weights (N4096 M=1: INT8 6.83 -> 5.68 us, INT2 5.88 -> 5.35 us; INT4 stays
// at four, 7.76 against 7.87 us with two).
template <int S, int MT>
constexpr int a8_rows() { return MT >= 8 || (MT == 1 && S != UQ_INT4) ? 2 : 4; }
constexpr int kA8Block = 32768;     // activation codes staged per LDS block (all rows of x together)

template <int S>
struct A8 {
  static constexpr int bits = Fmt<S>::bits;
  static constexpr int CPC = 128 / bits;      // codes per 16-byte chunk: 16, 32, 64
  static constexpr int CPD = 32 / bits;       // codes per dword: 4, 8, 16
  // 16-byte chunks per lane and row in flight: a whole row of K = 4096 per wave.
  static constexpr int CHUNKS = bits / 2;
};

// Position of code i (0..15) of a 16-code unit in the LDS order of the
// unpacked weight lanes.
template <int S>
__device__ __forceinline__ int a8_slot(int i) {
  if constexpr (S == UQ_INT8) return i;
  else if constexpr (S == UQ_INT4) return (i & 8) + (i & 1) * 4 + ((i & 7) >> 1);  // evens, then odds
  else return (i & 3) * 4 + (i >> 2);                                            // crumb j of each byte
}

// Quantize the 16 values of one unit with the group's max |x| (R-AQ): fp32
// division 127 / a, fp32 product, round to nearest even, clamp.
__device__ __forceinline__ void quantize16(const float (&v)[16], float a, int (&q)[16]) {
  const float r = a > 0.0f ? 127.0f / a : 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float t = __builtin_rintf(v[i] * r);
    t = t > 127.0f ? 127.0f : (t < -127.0f ? -127.0f : t);
    q[i] = int(t);
  }
}

// One unit's 16 fp16 values (two 16-byte loads) as fp32, and their max |x|.
__device__ __forceinline__ float unpack16(const uint4& a, const uint4& b, float (&v)[16]) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  float mx = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = h2f(uint16_t(w[i] & 0xFFFFu));
    v[2 * i + 1] = h2f(uint16_t(w[i] >> 16));
    mx = fmaxf(mx, fmaxf(fabsf(v[2 * i]), fabsf(v[2 * i + 1])));
  }
  return mx;
}

__device__ __forceinline__ float load16(const uint16_t* p, float (&v)[16]) {
  return unpack16(reinterpret_cast<const uint4*>(p)[0], reinterpret_cast<const uint4*>(p)[1], v);
}

// Max over the G/16 consecutive lanes that hold one group's units.
template <int G>
__device__ __forceinline__ float group_max(float a) {
#pragma unroll
  for (int o = 1; o < G / 16; o <<= 1) a = fmaxf(a, __shfl_xor(a, o));
  return a;
}

__device__ __forceinline__ float wave_total(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int S, int G, int MT>
__global__ __launch_bounds__(kA8Threads) void gemv_a8_kernel(const uint8_t* __restrict__ codes,
                                                              const uint8_t* __restrict__ params,
                                                              const uint16_t* __restrict__ x,
                                                              float* __restrict__ y, int n, int k, int m,
                                                              int kb_max) {
  using F = A8<S>;
  constexpr int CPC = F::CPC, CPD = F::CPD;
  constexpr int FU = G < CPC ? G : CPC;          // codes per scaled portion
  constexpr int NFU = CPC / FU;                  // portions per chunk
  constexpr int DPF = FU / CPD;                  // dwords per portion
  constexpr int UPF = FU / 16;                   // 16-code units per portion
  constexpr int kA8Chunks = F::CHUNKS;
  constexpr int kA8Rows = a8_rows<S, MT>();

  extern __shared__ uint4 a8_lds[];
  int8_t* qx = reinterpret_cast<int8_t*>(a8_lds);                      // [MT][kb_max]
  int* qsum = reinterpret_cast<int*>(qx + size_t(MT) * kb_max);        // [MT][kb_max / 16]
  float* sxs = reinterpret_cast<float*>(qsum + MT * (kb_max / 16));    // [MT][kb_max / G]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row0 = (blockIdx.x * kA8Waves + wave) * kA8Rows;
  const size_t rowb = size_t(k) * Fmt<S>::bits / 8;
  const int ng = k / G;
  int rr[kA8Rows];
#pragma unroll
  for (int r = 0; r < kA8Rows; ++r) rr[r] = row0 + r < n ? row0 + r : n - 1;  // past N: computed, not stored

  float acc_y[kA8Rows][MT];
#pragma unroll
  for (int r = 0; r < kA8Rows; ++r)
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) acc_y[r][mm] = 0.0f;

  // Loads of one batch of kA8Chunks chunks per lane and row (and their group
  // parameters); chunks past the block re-read a valid one and are skipped.
  uint4 cw[kA8Chunks][kA8Rows];
  uint32_t pw[kA8Chunks][kA8Rows][NFU];
  auto load_batch = [&](const uint8_t* cblk, int kb0, int cb, int nch) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kA8Chunks; ++j) {
      const int c0 = cb + j * 64 + lane;
      const int c = c0 < nch ? c0 : nch - 1;
#pragma unroll
      for (int r = 0; r < kA8Rows; ++r) {
        cw[j][r] = reinterpret_cast<const uint4*>(cblk + size_t(rr[r]) * rowb)[c];
#pragma unroll
        for (int f = 0; f < NFU; ++f) {
          const int g = (kb0 + c * CPC + f * FU) / G;
          pw[j][r][f] = reinterpret_cast<const uint32_t*>(params + size_t(rr[r]) * size_t(ng) * 4)[g];
        }
      }
    }
  };

  for (int kb0 = 0; kb0 < k; kb0 += kb_max) {
    const int kb = k - kb0 < kb_max ? k - kb0 : kb_max;
    const int upr = kb / 16;  // units per activation row in this block
    const int nch = kb / CPC;  // chunks per row in the block (kb is a multiple of CPC)
    const uint8_t* cblk = codes + size_t(kb0) * Fmt<S>::bits / 8;
    __syncthreads();          // the previous block's codes are no longer read
    // Stage: quantize each activation row of the block (rows past m: zeros).
    // The first unit's activations are loaded before the first batch of
    // weight loads, which then stay in flight while the units are quantized
    // (loads complete in order: using the activations waits for them only).
    for (int u0 = 0; u0 < MT * upr; u0 += kA8Threads) {
      const int u = u0 + tid;
      const bool valid = u < MT * upr;
      const int mm = valid ? u / upr : 0, ul = valid ? u % upr : 0;
      // Raw loads first (rows past m read row 0 and are zeroed below), then the
      // first weight batch, then the conversion that waits for the raw loads.
      const bool live = valid && mm < m;
      const uint4* xp = reinterpret_cast<const uint4*>(x + (live ? size_t(mm) * k + kb0 + ul * 16 : 0));
      const uint4 xa = xp[0], xb = xp[1];
      if (u0 == 0) load_batch(cblk, kb0, 0, nch);
      float v[16];
      float a = unpack16(live ? xa : make_uint4(0u, 0u, 0u, 0u), live ? xb : make_uint4(0u, 0u, 0u, 0u), v);
      a = group_max<G>(a);  // every lane takes part (G/16 divides 64 and upr)
      if (valid) {
        int q[16];
        quantize16(v, a, q);
        int sum = 0;
        uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sum += q[i];
          const int sl = a8_slot<S>(i);
          packed[sl >> 2] |= (uint32_t(q[i]) & 0xFFu) << (8 * (sl & 3));
        }
        reinterpret_cast<uint4*>(qx + size_t(mm) * kb_max)[ul] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        qsum[mm * (kb_max / 16) + ul] = sum;
        if ((ul * 16) % G == 0) sxs[mm * (kb_max / G) + (ul * 16) / G] = a / 127.0f;
      }
    }
    __syncthreads();

    // Stream the rows' codes of this block in batches of kA8Chunks chunks per lane.
    for (int cb = 0; cb < nch; cb += 64 * kA8Chunks) {
      if (cb > 0) load_batch(cblk, kb0, cb, nch);
#pragma unroll
      for (int j = 0; j < kA8Chunks; ++j) {
        const int c = cb + j * 64 + lane;
        if (c >= nch) continue;
#pragma unroll
        for (int f = 0; f < NFU; ++f) {
          const int kl = c * CPC + f * FU;  // first code of the portion within the block
          const int g = kl / G;             // group within the block (blocks start on group bounds)
          // Activation codes of the portion, and their sums and scales, per activation row.
          int qv[MT][DPF * (CPD / 4)];
          int qs[MT];
          float sx[MT];
#pragma unroll
          for (int mm = 0; mm < MT; ++mm) {
#pragma unroll
            for (int d = 0; d < UPF; ++d) {
              const uint4 t = reinterpret_cast<const uint4*>(qx + size_t(mm) * kb_max + kl)[d];
              qv[mm][4 * d] = int(t.x);
              qv[mm][4 * d + 1] = int(t.y);
              qv[mm][4 * d + 2] = int(t.z);
              qv[mm][4 * d + 3] = int(t.w);
            }
            int s = 0;
#pragma unroll
            for (int d = 0; d < UPF; ++d) s += qsum[mm * (kb_max / 16) + kl / 16 + d];
            qs[mm] = s;
            sx[mm] = sxs[mm * (kb_max / G) + g];
          }
#pragma unroll
          for (int r = 0; r < kA8Rows; ++r) {
            const uint32_t cw4[4] = {cw[j][r].x, cw[j][r].y, cw[j][r].z, cw[j][r].w};
            int dacc[MT];
#pragma unroll
            for (int mm = 0; mm < MT; ++mm) dacc[mm] = 0;
#pragma unroll
            for (int d = 0; d < DPF; ++d) {
              const uint32_t w = cw4[f * DPF + d];
              if constexpr (S == UQ_INT8) {
                const int ws = int(w ^ 0x80808080u);  // q - 128 as signed bytes
#pragma unroll
                for (int mm = 0; mm < MT; ++mm) dacc[mm] = __builtin_amdgcn_sdot4(ws, qv[mm][d], dacc[mm], false);
              } else if constexpr (S == UQ_INT4) {
                const int lo = int(w & 0x0F0F0F0Fu), hi = int((w >> 4) & 0x0F0F0F0Fu);
#pragma unroll
                for (int mm = 0; mm < MT; ++mm) {
                  dacc[mm] = __builtin_amdgcn_sdot4(lo, qv[mm][2 * d], dacc[mm], false);
                  dacc[mm] = __builtin_amdgcn_sdot4(hi, qv[mm][2 * d + 1], dacc[mm], false);
                }
              } else {
#pragma unroll
                for (int cj = 0; cj < 4; ++cj) {
                  const int cr = int((w >> (2 * cj)) & 0x03030303u);
#pragma unroll
                  for (int mm = 0; mm < MT; ++mm) dacc[mm] = __builtin_amdgcn_sdot4(cr, qv[mm][4 * d + cj], dacc[mm], false);
                }
              }
            }
            const uint32_t p = pw[j][r][f];
            const float s = h2f(uint16_t(p & 0xFFFFu)), z = h2f(uint16_t(p >> 16));
#pragma unroll
            for (int mm = 0; mm < MT; ++mm) {
              const int dd = S == UQ_INT8 ? dacc[mm] + 128 * qs[mm] : dacc[mm];
              const float t = __builtin_fmaf(s, float(dd), z * float(qs[mm]));
              acc_y[r][mm] = __builtin_fmaf(sx[mm], t, acc_y[r][mm]);
            }
          }
        }
      }
    }
  }

#pragma unroll
  for (int r = 0; r < kA8Rows; ++r)
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
      const float v = wave_total(acc_y[r][mm]);
      if (lane == 0 && row0 + r < n && mm < m) y[size_t(mm) * size_t(n) + size_t(row0 + r)] = v;
    }
}

// Test hook: the activation quantization alone, codes in natural order.
template <int G>
__global__ __launch_bounds__(kA8Threads) void quantize_a8_kernel(const uint16_t* __restrict__ x,
                                                                 int8_t* __restrict__ q, float* __restrict__ sx,
                                                                 int k, int64_t units) {
  const int64_t u = int64_t(blockIdx.x) * kA8Threads + threadIdx.x;
  const bool valid = u < units;  // units never straddle rows (k is a multiple of 16)
  const int64_t uu = valid ? u : 0;
  float v[16];
  float a = load16(x + uu * 16, v);
  a = group_max<G>(a);  // the grid covers whole groups: units is a multiple of G / 16
  if (!valid) return;
  int qi[16];
  quantize16(v, a, qi);
  uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) packed[i >> 2] |= (uint32_t(qi[i]) & 0xFFu) << (8 * (i & 3));
  reinterpret_cast<uint4*>(q)[uu] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  if ((uu * 16) % G == 0) sx[(uu * 16) / G] = a / 127.0f;
}

template <int S, int G, int MT>
hipError_t launch_a8(const uq_layout* L, const void* codes, const void* params, const uint16_t* x, float* y,
                     int m, hipStream_t stream) {
  const int n = int(L->n), k = int(L->k);
  int kb_max = kA8Block / MT;
  if (kb_max > k) kb_max = k;
  const size_t shmem = size_t(MT) * kb_max + size_t(MT) * (kb_max / 16) * 4 + size_t(MT) * (kb_max / G) * 4;
  constexpr int R = a8_rows<S, MT>();
  const int64_t blocks = (int64_t(n) + kA8Waves * R - 1) / (kA8Waves * R);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const uint8_t* c8 = static_cast<const uint8_t*>(codes);
  const uint8_t* p8 = static_cast<const uint8_t*>(params);
  int mi = m;
  void* args[] = {&c8, &p8, (void*)&x, &y, (void*)&n, (void*)&k, &mi, &kb_max};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemv_a8_kernel<S, G, MT>), dim3(unsigned(blocks)),
                         dim3(kA8Threads), args, shmem, stream);
}

template <int S, int G>
hipError_t launch_a8_m(const uq_layout* L, const void* codes, const void* params, const uint16_t* x, float* y,
                       int m, hipStream_t stream) {
  if (m <= 1) return launch_a8<S, G, 1>(L, codes, params, x, y, m, stream);
  if (m <= 2) return launch_a8<S, G, 2>(L, codes, params, x, y, m, stream);
  if (m <= 4) return launch_a8<S, G, 4>(L, codes, params, x, y, m, stream);
  return launch_a8<S, G, 8>(L, codes, params, x, y, m, stream);
}

}  // namespace
}  // namespace uq

#include "gemv_a8_mfma.hpp"

namespace uq {
namespace {

// 2 to 8 activation rows (3 to 8 for INT2) on the integer matrix cores when
// the layout has a matrix-core form (INT4 / INT8 with groups of 32, 64 or
// 128, INT2 with groups of 16) and the shape fits (judged at eight rows, so
// every such M takes the same kernel), else the dot-product kernel.  Eight
// waves per workgroup, each an eighth of every row.  Measured on MI355X
// (graph replay): INT8 G128 N4096 M=8 18.7 -> 8.0 us, INT4 G64 N11008 M=4
// 16.9 -> 11.3 us when first moved; a single row stays on the dot-product
// kernel (INT8 5.8 against 6.0 us, INT4 7.8 against 8.8).
template <int S, int G>
hipError_t launch_a8_sel(const uq_layout* L, const void* codes, const void* params, const uint16_t* x, float* y,
                         int m, hipStream_t stream) {
  if constexpr (a8_mfma_scheme<S, G>()) {
    constexpr int W = 8;
    // Measured on MI355X against the dot product: INT4 G32 N11008 M=2 / 3 / 4
    // / 8 10.9 / 16.7 / 16.9 / 43.6 -> 9.6 / 11.4 / 12.0 / 14.7 us, INT8 G32
    // N4096 M=2 / 4 / 8 9.1 / 13.1 / 18.4 -> 7.3 / 7.9 / 8.5 us; INT2 G16 pays
    // off from three rows (N4096 M=2 / 3 / 8 7.6 / 11.5 / 18.3 -> 7.7 / 8.4 /
    // 8.7 us).
    constexpr int min_rows = S == UQ_INT2 ? 3 : 2;
    if (m >= min_rows && a8m_fits<S, G>(L->k, 8, W)) {
      if (m <= 2) return launch_a8m_w<S, G, 2, W>(L, codes, params, x, y, m, stream);
      if (m <= 4) return launch_a8m_w<S, G, 4, W>(L, codes, params, x, y, m, stream);
      return launch_a8m_w<S, G, 8, W>(L, codes, params, x, y, m, stream);
    }
  }
  return launch_a8_m<S, G>(L, codes, params, x, y, m, stream);
}

template <int G>
hipError_t launch_quantize(const uint16_t* x, int8_t* q, float* sx, int64_t m, int k, hipStream_t stream) {
  const int64_t units = m * (k / 16);
  const int64_t blocks = (units + kA8Threads - 1) / kA8Threads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  void* args[] = {(void*)&x, &q, &sx, &k, (void*)&units};
  return hipLaunchKernel(reinterpret_cast<const void*>(&quantize_a8_kernel<G>), dim3(unsigned(blocks)),
                         dim3(kA8Threads), args, 0, stream);
}

}  // namespace

hipError_t launch_gemv_a8(const uq_layout* L, const void* codes, const void* params, const uint16_t* x,
                          float* y, int m, hipStream_t stream) {
  switch (L->scheme * 1000 + L->group) {
    case UQ_INT2 * 1000 + 16: return launch_a8_sel<UQ_INT2, 16>(L, codes, params, x, y, m, stream);
    case UQ_INT2 * 1000 + 32: return launch_a8_sel<UQ_INT2, 32>(L, codes, params, x, y, m, stream);
    case UQ_INT2 * 1000 + 64: return launch_a8_sel<UQ_INT2, 64>(L, codes, params, x, y, m, stream);
    case UQ_INT2 * 1000 + 128: return launch_a8_sel<UQ_INT2, 128>(L, codes, params, x, y, m, stream);
    case UQ_INT4 * 1000 + 32: return launch_a8_sel<UQ_INT4, 32>(L, codes, params, x, y, m, stream);
    case UQ_INT4 * 1000 + 64: return launch_a8_sel<UQ_INT4, 64>(L, codes, params, x, y, m, stream);
    case UQ_INT4 * 1000 + 128: return launch_a8_sel<UQ_INT4, 128>(L, codes, params, x, y, m, stream);
    case UQ_INT8 * 1000 + 32: return launch_a8_sel<UQ_INT8, 32>(L, codes, params, x, y, m, stream);
    case UQ_INT8 * 1000 + 64: return launch_a8_sel<UQ_INT8, 64>(L, codes, params, x, y, m, stream);
    case UQ_INT8 * 1000 + 128: return launch_a8_sel<UQ_INT8, 128>(L, codes, params, x, y, m, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_quantize_a8(int32_t group, const uint16_t* x, int8_t* q, float* sx, int64_t m, int64_t k,
                              hipStream_t stream) {
  switch (group) {
    case 16: return launch_quantize<16>(x, q, sx, m, int(k), stream);
    case 32: return launch_quantize<32>(x, q, sx, m, int(k), stream);
    case 64: return launch_quantize<64>(x, q, sx, m, int(k), stream);
    case 128: return launch_quantize<128>(x, q, sx, m, int(k), stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace uq
