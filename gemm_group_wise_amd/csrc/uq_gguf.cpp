// GGUF Q4_0 / Q8_0 weight blocks re-laid into the library's INT layout.
//
// The "Ultra LLM Engine" page lists dequantizers for the GGUF block formats
// Q4_0 and Q8_0 on its roadmap (Roadmap Ideas) and has its loader refuse
// tensors it cannot decode rather than guess (Checkpoint Loading).  The block
// layout is the public GGUF one: 32 consecutive weights of a row per block,
// an fp16 scale d first; Q4_0 then holds 16 bytes whose low nibbles are
// weights 0..15 and high nibbles weights 16..31, each (nibble - 8) * d; Q8_0
// holds 32 signed bytes, each q * d.
//
// Both are group-wise affine codes with G = 32, so they map exactly onto the
// INT form w' = q * s + z: Q4_0 as INT4 (q = nibble, s = d, z = -8 d) and
// Q8_0 as INT8 (q = byte ^ 0x80, i.e. the signed value + 128, s = d,
// z = -128 d).  z is a power-of-two multiple of d, exact in fp16 unless it
// overflows; such blocks, and non-finite scales, are refused.  The GEMV,
// GEMM and dequant kernels then serve the imported weights unchanged.  The
// re-layout happens once, on the host, when weights are loaded: the kernels
// keep their 16-byte-chunk code rows and separate parameter rows instead of
// reading 18- and 34-byte blocks that no vector load can align to.
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "uq_internal.h"

namespace uq {
namespace {

constexpr int kBlock = 32;

int block_bytes(int32_t type) { return type == UQ_GGUF_Q4_0 ? 18 : 34; }

uint16_t load_le16(const uint8_t* p) { return uint16_t(p[0] | (uint32_t(p[1]) << 8)); }

// -(2^shift) * d as fp16 bits, for a finite fp16 d (bits h) whose product
// stays within the fp16 range.  Scaling by a power of two is exact: a normal
// d only moves its exponent; a subnormal d = m * 2^-24 shifts its integer
// significand left and, past 10 bits, turns normal.
uint16_t neg_pow2_times(uint16_t h, int shift) {
  const uint16_t sign = uint16_t((h & 0x8000u) ^ 0x8000u);
  const uint32_t e = (h >> 10) & 0x1fu, mant = h & 0x3ffu;
  if (e == 0 && mant == 0) return sign;             // +-0 -> -+0
  if (e != 0) return uint16_t(sign | ((e + shift) << 10) | mant);
  uint32_t m = mant << shift;                       // subnormal: m * 2^-24
  if (m < 0x400u) return uint16_t(sign | m);
  uint32_t ex = 1;                                  // normalize: hidden bit at 0x400
  while (m >= 0x800u) { m >>= 1; ++ex; }            // exact: m has at most 10 + shift bits, low bits zero
  return uint16_t(sign | (ex << 10) | (m & 0x3ffu));
}

// Largest |d| whose z = -(2^shift) d fits fp16 (65504 = 0x7BFF), as fp16 bits.
bool zero_fits(uint16_t h, int shift) {
  const uint32_t e = (h >> 10) & 0x1fu;
  if (e == 0x1fu) return false;                     // inf or NaN scale
  if (e == 0) return true;                          // subnormal * 2^shift <= 2^-14 * 2^7 < 65504
  return e + uint32_t(shift) <= 30u;                // largest finite exponent field is 30
}

void relayout_rows(int32_t type, const uint8_t* src, int64_t k, uint8_t* codes, uint16_t* params,
                   int64_t r0, int64_t r1) {
  const int64_t nb = k / kBlock;
  const int bb = block_bytes(type);
  const int shift = type == UQ_GGUF_Q4_0 ? 3 : 7;
  const size_t row_codes = type == UQ_GGUF_Q4_0 ? size_t(k) / 2 : size_t(k);
  for (int64_t r = r0; r < r1; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const uint8_t* blk = src + (size_t(r) * size_t(nb) + size_t(b)) * size_t(bb);
      const uint16_t d = load_le16(blk);
      const uint8_t* qs = blk + 2;
      uint16_t* pr = params + (size_t(r) * size_t(nb) + size_t(b)) * 2;
      pr[0] = d;
      pr[1] = neg_pow2_times(d, shift);
      if (type == UQ_GGUF_Q4_0) {
        // INT4 byte t holds weights 2t (low nibble) and 2t + 1 (high nibble)
        // of the group; weight i of the block is nibble i % 16 of byte i / 16.
        uint8_t* out = codes + size_t(r) * row_codes + size_t(b) * 16;
        auto nib = [qs](int i) { return i < 16 ? (qs[i] & 0x0fu) : (qs[i - 16] >> 4); };
        for (int t = 0; t < 16; ++t) out[t] = uint8_t(nib(2 * t) | (nib(2 * t + 1) << 4));
      } else {
        uint8_t* out = codes + size_t(r) * row_codes + size_t(b) * 32;
        for (int i = 0; i < 32; ++i) out[i] = uint8_t(qs[i] ^ 0x80u);
      }
    }
  }
}

}  // namespace

uq_status import_gguf(int32_t type, const void* blocks, int64_t n, int64_t k, uq_layout* L,
                      uint8_t* codes, uint16_t* params) {
  if (!blocks || !L || !codes || !params) return UQ_ERR_NULL;
  if (type != UQ_GGUF_Q4_0 && type != UQ_GGUF_Q8_0) return UQ_ERR_UNSUPPORTED;
  uq_layout lay;
  lay.scheme = type == UQ_GGUF_Q4_0 ? UQ_INT4 : UQ_INT8;
  lay.group = kBlock;
  lay.n = n;
  lay.k = k;
  const uq_status st = check_layout(&lay);
  if (st != UQ_OK) return st;

  const uint8_t* src = static_cast<const uint8_t*>(blocks);
  const size_t nblocks = size_t(n) * size_t(k / kBlock);
  const int bb = block_bytes(type);
  const int shift = type == UQ_GGUF_Q4_0 ? 3 : 7;
  for (size_t i = 0; i < nblocks; ++i)             // validate every scale before writing
    if (!zero_fits(load_le16(src + i * size_t(bb)), shift)) return UQ_ERR_RANGE;

  unsigned nt = std::thread::hardware_concurrency();
  nt = nt == 0 ? 1 : (nt > 16 ? 16 : nt);
  if (size_t(n) * size_t(k) < (size_t(1) << 20)) nt = 1;
  if (nt == 1) {
    relayout_rows(type, src, k, codes, params, 0, n);
  } else {
    std::vector<std::thread> th;
    const int64_t step = (n + nt - 1) / nt;
    for (unsigned t = 0; t < nt; ++t) {
      const int64_t r0 = int64_t(t) * step, r1 = r0 + step < n ? r0 + step : n;
      if (r0 >= r1) break;
      th.emplace_back(relayout_rows, type, src, k, codes, params, r0, r1);
    }
    for (auto& t : th) t.join();
  }
  *L = lay;
  return UQ_OK;
}

}  // namespace uq
