// Internal definitions shared by the host packer, the C ABI and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "uq.h"

namespace uq {

// NormalFloat4 codebook (QLoRA construction: standard-normal quantiles at
// 8 equally spaced probabilities from p* = 0.9677083 down to 0.5 for the
// positive side, 7 for the negative side, plus 0, scaled to [-1, 1]); fp32
// bit patterns, index 0 -> 15.  "Ultra LLM Engine", Core Components >
// Quantization, nf4 row.
static constexpr uint32_t kNf4Bits[16] = {
    0xbf800000u, 0xbf3239b3u, 0xbf066b30u, 0xbeca32a0u,
    0xbe91a24cu, 0xbe3d353fu, 0xbdba786bu, 0x00000000u,
    0x3da2fb03u, 0x3e24cae1u, 0x3e7c04dcu, 0x3ead0338u,
    0x3ee1a4b7u, 0x3f1007aau, 0x3f3913b1u, 0x3f800000u};

// Code width in bits per scheme; 0 for an unknown scheme.
constexpr int scheme_bits(int scheme) {
  return scheme == UQ_INT2 ? 2
       : scheme == UQ_INT4 ? 4
       : scheme == UQ_INT8 ? 8
       : scheme == UQ_NF4  ? 4
                           : 0;
}

constexpr bool group_supported(int scheme, int g) {
  return scheme == UQ_INT2 ? (g == 16 || g == 32 || g == 64 || g == 128)
       : scheme == UQ_INT4 ? (g == 32 || g == 64 || g == 128)
       : scheme == UQ_INT8 ? (g == 32 || g == 64 || g == 128)
       : scheme == UQ_NF4  ? (g == 64)
                           : false;
}

// Bytes of one group's parameters: (s, z) fp16 pair, or one fp16 absmax.
constexpr int param_bytes_per_group(int scheme) { return scheme == UQ_NF4 ? 2 : 4; }

constexpr int64_t kMaxK = int64_t(1) << 24;
constexpr int64_t kMaxN = 0x7fffffff;

// Shape/format validation common to every entry point.
inline uq_status check_layout(const uq_layout* L) {
  if (!L) return UQ_ERR_NULL;
  const int bits = scheme_bits(L->scheme);
  if (!bits) return UQ_ERR_UNSUPPORTED;
  if (!group_supported(L->scheme, L->group)) return UQ_ERR_UNSUPPORTED;
  if (L->n < 1 || L->n > kMaxN) return UQ_ERR_SHAPE;
  if (L->k < 1 || L->k > kMaxK) return UQ_ERR_SHAPE;
  if (L->k % L->group) return UQ_ERR_SHAPE;
  if ((L->k * bits) % 128) return UQ_ERR_SHAPE;  // whole 16-byte code chunks
  return UQ_OK;
}

inline size_t code_row_bytes(const uq_layout* L) {
  return size_t(L->k) * size_t(scheme_bits(L->scheme)) / 8;
}
inline size_t param_row_bytes(const uq_layout* L) {
  return size_t(L->k / L->group) * size_t(param_bytes_per_group(L->scheme));
}

// ---- GEMM plan and workspace (shared by the launcher and the host-side
// validation, so the size a caller is told to allocate is the size used) ----

constexpr int kGemmMaxSplit = 4;              // workgroups one tile's K steps may be split over
constexpr int64_t kGemmMaxSplitTiles = 16384; // tiles that can have a K split (one counter each)
constexpr int64_t kGemmMinTiles = 128;        // grids below this take the next smaller row tile

// Tilings: 8 waves (two per SIMD); BM rows of x by BN = 64 * wgn weight rows.
// The largest tile that fits M is the cheapest per output (each dequantized
// fragment feeds BM / 32 M tiles) as long as the grid still gives at least
// half of the 256 CUs a workgroup; a narrower weight matrix takes the next
// smaller tile instead (N = 4096, M = 256: 64 workgroups of 128 rows took
// 49.6 us, 256 of 64 rows 28.3 us; at N = 11008 the 172 large tiles beat 688
// small ones, 47.8 against 64.8 us).  (A 256-row tile on 4 waves, one per
// SIMD with the accumulators in AGPRs, halves the dequant work per MFMA but
// measured slower: a lone wave per SIMD hides neither the copies' waits nor
// the LDS latency.)  Up to 64 rows a workgroup's time is mostly the latency
// of its K steps (each waits for copies issued one or two steps earlier), so
// the K steps of a tile may be split over up to kGemmMaxSplit workgroups
// (the launcher picks the count from the kernel's occupancy).  Measured per
// call: INT8 / INT2 at N = 4096, M = 64 (64 tiles) 27.1 / 25.4 us unsplit,
// 14.5 / 14.3 us in four; INT4 at N = 11008 (172 tiles, one workgroup per CU)
// M = 16 16.4 us unsplit against 22.1 / 24.1 us in two / four, and M = 64
// 22.6 us on 64-row tiles against 30.4 us on 344 tiles of 32 rows.
struct GemmPlan {
  int bm, wgn, ksplit;
  bool xf;  // the GEMM stages the caller's fp16 x and rounds it to bf16 itself
};

// Above 64 rows on 64-row tiles, INT8 and INT2 (whose dequant leaves room in
// the VALU budget) also stage the caller's fp16 x and round it themselves,
// which saves the conversion launch (measured on MI355X, N = 4096: INT8 M =
// 80 / 128 / 256 25.3 / 25.7 / 26.9 -> 23.2 / 23.5 / 24.0 us, Q8_0-style
// INT8 G32 M = 256 28.0 -> 24.7 us, INT2 M = 256 23.9 -> 22.5 us),
// while INT4 and NF4 measured slower that way (INT4 N = 11008 M = 128 37.3
// -> 38.0 us, NF4 N = 14336 M = 128 47.2 -> 50.4 us).
inline GemmPlan plan_gemm(int64_t m, int64_t n, int32_t scheme) {
  auto tiles = [&](int64_t bm, int64_t bn) { return ((m + bm - 1) / bm) * ((n + bn - 1) / bn); };
  if (m > 64 && tiles(128, 128) >= kGemmMinTiles) return {128, 2, 1, false};
  if (m > 64) return {64, 1, 1, scheme == UQ_INT8 || scheme == UQ_INT2};
  if (m > 32) return {64, 1, 1, true};
  return {32, 1, 1, true};
}

// Byte offsets of the regions of a uq_gemm workspace and its total size.
// Regions start on 256-byte boundaries.  The partial tiles are sized for the
// largest K split (kGemmMaxSplit), so the size does not depend on the device.
struct GemmWorkspace {
  size_t counters;  // kGemmMaxSplitTiles uint32 arrival counters (zero between calls)
  size_t act;       // bf16 x [m rounded up to 128][k] (empty when the GEMM reads fp16 x)
  size_t part;      // fp32 partial tiles [kGemmMaxSplit][m rounded up to the row tile][n]
  size_t total;
};

inline GemmWorkspace gemm_workspace(const uq_layout* L, int64_t m) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  const GemmPlan p = plan_gemm(m, L->n, L->scheme);
  GemmWorkspace w;
  w.counters = 0;
  w.act = up(size_t(kGemmMaxSplitTiles) * 4);
  const size_t act_bytes = p.xf ? 0 : size_t((m + 127) / 128 * 128) * size_t(L->k) * 2;
  w.part = up(w.act + act_bytes);
  const size_t part_bytes =
      p.bm <= 64 ? size_t(kGemmMaxSplit) * size_t((m + p.bm - 1) / p.bm * p.bm) * size_t(L->n) * 4 : 0;
  w.total = up(w.part + part_bytes);
  return w;
}

// Size of the fixed device scratch uq_gemm_noalloc works in (one per GPU).
constexpr size_t kGemmScratchBytes = size_t(UQ_GEMM_NOALLOC_MAX_BYTES);

// ---- Argument checks of the device entry points (uq_check.cpp; host only,
// no HIP call) ----
uq_status check_product(const uq_layout* L, const void* codes, const void* params, const void* x,
                        const void* y, int64_t m, int64_t mmax);
uq_status check_gemm_workspace(const uq_layout* L, int64_t m, const void* workspace, size_t bytes);
uq_status check_dequant(const uq_layout* L, const void* codes, const void* params, const void* w);
uq_status check_quantize_activations(int32_t group, const void* x, const void* q, const void* sx, int64_t m,
                                     int64_t k);
uq_status check_rmsnorm_rope(const void* x, const void* y, const void* gamma, const void* pos, const void* cos,
                             const void* sin, int64_t tokens, int32_t heads, int32_t head_dim, int64_t max_pos,
                             float eps);
uq_status check_probe_read(const void* src, size_t bytes, int32_t workgroups, int32_t loads_in_flight,
                           const void* sink);

// Host packer (uq_pack.cpp).
uq_status pack_weights(const uq_layout* L, const float* w, uint8_t* codes,
                       uint16_t* params);

// Host re-layout of GGUF Q4_0 / Q8_0 blocks into the INT4 / INT8 G = 32 layout (uq_gguf.cpp).
uq_status import_gguf(int32_t type, const void* blocks, int64_t n, int64_t k, uq_layout* L,
                      uint8_t* codes, uint16_t* params);

// Host rotary table (rope_table.cpp).
uq_status rope_table(double theta, int32_t head_dim, int64_t max_pos, float* cos_out, float* sin_out);

// Head dimensions the fused RMSNorm + RoPE kernel serves.
constexpr bool rope_head_dim_supported(int32_t d) { return d == 64 || d == 128 || d == 256 || d == 512; }

}  // namespace uq
