// Host-side quantizer and packer ("Ultra LLM Engine", Core Components >
// Quantization: group-wise asymmetric INT-N and NF4, codes packed into bytes).
//
// Built with -ffp-contract=off and without fast-math: every fp32 and fp64
// operation below is one IEEE operation rounded to nearest even, which is
// what makes the packed bytes reproducible bit for bit.
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "uq_internal.h"

namespace uq {
namespace {

// fp32 -> fp16 bit pattern, round to nearest, ties to even (IEEE 754
// convertFormat).  Handles subnormal results; inputs here are finite and
// within +-65504 (validated by the caller), but overflow still rounds to inf.
uint16_t f32_to_f16(float f) {
  uint32_t x;
  std::memcpy(&x, &f, 4);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7fffffffu;
  if (ax >= 0x7f800000u) return uint16_t(sign | 0x7c00u | (ax > 0x7f800000u ? 0x200u : 0u));
  if (ax >= 0x38800000u) {  // |f| >= 2^-14: normal fp16 (or overflow)
    const uint32_t mant = ax & 0x7fffffu;
    const uint32_t exp = (ax >> 23) - 127 + 15;
    if (exp >= 31) return uint16_t(sign | 0x7c00u);
    uint32_t h = (exp << 10) | (mant >> 13);
    const uint32_t rem = mant & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ++h;  // carry may reach inf
    return uint16_t(sign | h);
  }
  if (ax < 0x33000000u) return uint16_t(sign);  // below 2^-25: rounds to zero
  // Subnormal result: units of 2^-24.  value = mant * 2^(e - 150).
  const uint32_t e = ax >> 23;
  const uint32_t mant = (ax & 0x7fffffu) | 0x800000u;
  const uint32_t shift = 126 - e;  // 14 .. 24
  uint32_t h = mant >> shift;
  const uint32_t rem = mant & ((1u << shift) - 1u);
  const uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (h & 1u))) ++h;
  return uint16_t(sign | h);
}

// fp16 bit pattern -> exact double.
double f16_to_f64(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int exp = (h >> 10) & 0x1f;
  const int mant = h & 0x3ff;
  double v;
  if (exp == 0) v = std::ldexp(double(mant), -24);
  else v = std::ldexp(double(mant | 0x400), exp - 25);
  return sign ? -v : v;
}

float nf4_entry(int i) {
  float f;
  std::memcpy(&f, &kNf4Bits[i], 4);
  return f;
}

// Quantize rows [r0, r1) of an INT-N matrix.
void pack_int_rows(const uq_layout* L, const float* w, uint8_t* codes,
                   uint16_t* params, int64_t r0, int64_t r1) {
  const int bits = scheme_bits(L->scheme);
  const int qmax = (1 << bits) - 1;
  const int64_t k = L->k, G = L->group, ng = k / G;
  const size_t rowb = code_row_bytes(L);
  std::vector<uint8_t> q(static_cast<size_t>(k));
  for (int64_t r = r0; r < r1; ++r) {
    const float* wr = w + size_t(r) * size_t(k);
    for (int64_t g = 0; g < ng; ++g) {
      const float* wg = wr + g * G;
      float mn = wg[0], mx = wg[0];
      for (int64_t i = 1; i < G; ++i) {
        mn = wg[i] < mn ? wg[i] : mn;
        mx = wg[i] > mx ? wg[i] : mx;
      }
      const float span = mx - mn;                    // fp32, one rounding
      const float s32 = span / float(qmax);          // fp32, one rounding
      const uint16_t s16 = f32_to_f16(s32);
      const uint16_t z16 = f32_to_f16(mn);
      const double sd = f16_to_f64(s16), zd = f16_to_f64(z16);
      uint8_t* qg = q.data() + g * G;
      if ((s16 & 0x7fffu) == 0) {
        std::memset(qg, 0, size_t(G));
      } else {
        for (int64_t i = 0; i < G; ++i) {
          const double d = (double(wg[i]) - zd) / sd;  // fp64
          double qi = std::nearbyint(d);               // ties to even
          qi = qi < 0.0 ? 0.0 : (qi > double(qmax) ? double(qmax) : qi);
          qg[i] = uint8_t(qi);
        }
      }
      params[(size_t(r) * size_t(ng) + size_t(g)) * 2 + 0] = s16;
      params[(size_t(r) * size_t(ng) + size_t(g)) * 2 + 1] = z16;
    }
    uint8_t* cr = codes + size_t(r) * rowb;
    const int per = 8 / bits;
    for (size_t j = 0; j < rowb; ++j) {
      uint32_t b = 0;
      for (int i = 0; i < per; ++i) b |= uint32_t(q[j * per + i]) << (bits * i);
      cr[j] = uint8_t(b);
    }
  }
}

// Quantize rows [r0, r1) of an NF4 matrix.
void pack_nf4_rows(const uq_layout* L, const float* w, uint8_t* codes,
                   uint16_t* params, int64_t r0, int64_t r1) {
  const int64_t k = L->k, G = L->group, ng = k / G;
  const size_t rowb = code_row_bytes(L);
  double mid[15];
  for (int i = 0; i < 15; ++i) mid[i] = (double(nf4_entry(i)) + double(nf4_entry(i + 1))) / 2.0;
  std::vector<uint8_t> q(static_cast<size_t>(k));
  for (int64_t r = r0; r < r1; ++r) {
    const float* wr = w + size_t(r) * size_t(k);
    for (int64_t g = 0; g < ng; ++g) {
      const float* wg = wr + g * G;
      float amax = 0.0f;
      for (int64_t i = 0; i < G; ++i) {
        const float a = std::fabs(wg[i]);
        amax = a > amax ? a : amax;
      }
      const uint16_t a16 = f32_to_f16(amax);
      const double ad = f16_to_f64(a16);
      uint8_t* qg = q.data() + g * G;
      for (int64_t i = 0; i < G; ++i) {
        if (ad == 0.0) { qg[i] = 7; continue; }
        const double v = double(wg[i]) / ad;
        int c = 0;
        while (c < 15 && v > mid[c]) ++c;  // midpoint stays with the lower entry
        qg[i] = uint8_t(c);
      }
      params[size_t(r) * size_t(ng) + size_t(g)] = a16;
    }
    uint8_t* cr = codes + size_t(r) * rowb;
    for (size_t j = 0; j < rowb; ++j) cr[j] = uint8_t(q[2 * j] | (q[2 * j + 1] << 4));
  }
}

}  // namespace

uq_status pack_weights(const uq_layout* L, const float* w, uint8_t* codes,
                       uint16_t* params) {
  const uq_status st = check_layout(L);
  if (st != UQ_OK) return st;
  if (!w || !codes || !params) return UQ_ERR_NULL;
  const size_t total = size_t(L->n) * size_t(L->k);
  for (size_t i = 0; i < total; ++i) {
    const float v = w[i];
    if (!(std::fabs(v) <= 65504.0f)) return UQ_ERR_RANGE;  // also rejects NaN
  }

  const int64_t n = L->n;
  unsigned nt = std::thread::hardware_concurrency();
  nt = nt == 0 ? 1 : (nt > 16 ? 16 : nt);
  if (total < (size_t(1) << 20)) nt = 1;
  auto work = [&](int64_t r0, int64_t r1) {
    if (L->scheme == UQ_NF4) pack_nf4_rows(L, w, codes, params, r0, r1);
    else pack_int_rows(L, w, codes, params, r0, r1);
  };
  if (nt == 1) {
    work(0, n);
  } else {
    std::vector<std::thread> th;
    const int64_t step = (n + nt - 1) / nt;
    for (unsigned t = 0; t < nt; ++t) {
      const int64_t r0 = int64_t(t) * step, r1 = r0 + step < n ? r0 + step : n;
      if (r0 >= r1) break;
      th.emplace_back(work, r0, r1);
    }
    for (auto& t : th) t.join();
  }
  return UQ_OK;
}

}  // namespace uq
