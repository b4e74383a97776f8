/*
 * uq.h -- C ABI of libuq: group-wise weight quantization and fused
 * dequant-GEMV / dequant-GEMM for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the "Ultra LLM Engine" page:
 *   - Core Components > Quantization (scheme table): group-wise asymmetric
 *     uniform INT-2/4/8 ("int") and NormalFloat4 with the QLoRA codebook
 *     ("nf4"); codes are packed several to a byte and come with matching
 *     dequantizers.
 *   - Core Components > Fused Kernels: a fused dequantized-weight GEMV for
 *     single-token decode and a fused dequantized-weight GEMM for batched
 *     decode.
 *   - Core Components > Quantized Model: linear layers keep their weights
 *     quantized (QuantLinear) and feed these products.
 *
 * Computation: y[m, n] = sum_k x[m, k] * w'[n, k], where w' is the
 * dequantized weight, x is fp16 and y is fp32 (fp32 accumulation).
 *
 * Arithmetic fixed by this library (the page states none of it):
 *   INT-N (b bits, qmax = 2^b - 1), per row n and group g of G consecutive k:
 *     s = fp16(fp32(fp32(max - min) / qmax)), z = fp16(min)      (RNE)
 *     q = clamp(rint((w - z) / s) in fp64, 0, qmax); q = 0 when s == 0
 *     w' = fp32(q * s + z)              (one rounding; equals one fp32 FMA)
 *   NF4 (G = 64): a = fp16(max |w|); q = nearest codebook entry to w / a
 *     (fp64; a value on a midpoint takes the lower index; a == 0 gives q = 7);
 *     w' = fp32(C[q] * a).
 *
 * Packed layout (what uq_pack_weights writes and the kernels read):
 *   codes  : uint8 [n][k * b / 8], row-major.  INT4/NF4: byte j holds code
 *            2j in bits 0-3 and code 2j+1 in bits 4-7.  INT2: byte j holds
 *            code 4j+i in bits 2i..2i+1.  INT8: one code per byte.
 *   params : INT-N: uint16 [n][k / G][2] = fp16 bit patterns (s, z)
 *            interleaved per group (as uint32 little-endian: s | z << 16).
 *            NF4:   uint16 [n][k / 64] = fp16 absmax bit patterns.
 *
 * Conventions for every call:
 *   - Validation runs before any HIP call.  On any status other than UQ_OK
 *     nothing was launched and no output was written.
 *   - The caller owns every buffer it passes.  Calls never synchronize:
 *     device work is enqueued on `stream` (a hipStream_t; NULL means the null
 *     stream) and the call returns at once.  Faults inside a kernel surface
 *     at the caller's next synchronization.  No call allocates device
 *     memory or keeps state between calls; uq_gemm works in a workspace the
 *     caller provides (see there).
 *   - Outputs are overwritten, never accumulated into.
 *   - All functions are thread-safe.
 */
#ifndef UQ_H
#define UQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum uq_status {
  UQ_OK = 0,
  UQ_ERR_NULL = 1,        /* a required pointer is NULL                      */
  UQ_ERR_SHAPE = 2,       /* n, k, m or group out of range, or k not a whole
                             number of groups and 16-byte code chunks        */
  UQ_ERR_UNSUPPORTED = 3, /* unknown scheme or unsupported (scheme, group)   */
  UQ_ERR_ALIGN = 4,       /* a device pointer is not suitably aligned        */
  UQ_ERR_RANGE = 5,       /* a weight is NaN, infinite, or |w| > 65504       */
  UQ_ERR_HIP = 6,         /* the HIP runtime rejected a kernel launch        */
  UQ_ERR_WORKSPACE = 7    /* a workspace is smaller than the call needs      */
} uq_status;

typedef enum uq_scheme {
  UQ_INT2 = 1, /* groups 16, 32, 64, 128 */
  UQ_INT4 = 2, /* groups 32, 64, 128     */
  UQ_INT8 = 3, /* groups 32, 64, 128     */
  UQ_NF4 = 4   /* group 64               */
} uq_scheme;

/* Shape and format of one quantized weight matrix W[n][k] (out x in). */
typedef struct uq_layout {
  int32_t scheme; /* a uq_scheme value                                   */
  int32_t group;  /* G: consecutive k sharing one (s, z) or one absmax   */
  int64_t n;      /* rows of W = output features, 1 .. 2^31 - 1          */
  int64_t k;      /* columns of W = input features; a multiple of G and
                     of the 16-byte chunk (128 / bits codes), <= 2^24    */
} uq_layout;

/* Limits. */
#define UQ_GEMV_MAX_M 8     /* uq_gemv serves 1..8 activation rows        */
#define UQ_GEMM_MAX_M 65536 /* uq_gemm serves 1..65536 activation rows    */

/* Sizes in bytes of the two packed arrays for `layout`.
 * Returns UQ_ERR_NULL / UQ_ERR_UNSUPPORTED / UQ_ERR_SHAPE on a bad layout. */
uq_status uq_packed_size(const uq_layout* layout, size_t* code_bytes,
                         size_t* param_bytes);

/* Quantize and pack W on the host (Core Components > Quantization).
 *   w      : host fp32 [n][k] row-major, finite with |w| <= 65504
 *   codes  : host, uq_packed_size code_bytes, written
 *   params : host, uq_packed_size param_bytes, written (uint16 fp16 bits)
 * Deterministic and pure.  UQ_ERR_RANGE if any weight is out of range
 * (checked before anything is written). */
uq_status uq_pack_weights(const uq_layout* layout, const float* w,
                          uint8_t* codes, uint16_t* params);

/* Fused dequant + GEMV for single-token and small-batch decode
 * (Core Components > Fused Kernels, GEMV during single-token decode):
 *   y[m][n] = sum_k x[m][k] * w'[n][k]   for 1 <= m <= UQ_GEMV_MAX_M
 *   codes, params : device, as packed by uq_pack_weights, 16-byte aligned
 *   x : device fp16 [m][k] row-major (uint16 bit patterns), 16-byte aligned
 *   y : device fp32 [m][n] row-major, 16-byte aligned, overwritten
 * The products are formed from fp16 activations with fp32 accumulation;
 * results match fp64 x . w'^T to within rounding (the NF4 codebook enters
 * the products as fp16 high and low parts, about 22 bits). */
uq_status uq_gemv(const uq_layout* layout, const void* codes,
                  const void* params, const uint16_t* x, float* y, int64_t m,
                  void* stream);

/* Bytes of device workspace uq_gemm needs for `layout` and m activation rows
 * (0 < m <= UQ_GEMM_MAX_M).  Host call; the size depends on (layout, m) only,
 * not on the device.  Errors as for uq_packed_size, UQ_ERR_SHAPE for m. */
uq_status uq_gemm_workspace_size(const uq_layout* layout, int64_t m, size_t* bytes);

/* Fused dequant + GEMM on the bf16 matrix cores for batched decode and
 * prefill (Core Components > Fused Kernels, GEMM during batched decode):
 *   y[m][n] = sum_k bf16(x[m][k]) * bf16(w'[n][k])  for 1 <= m <= UQ_GEMM_MAX_M
 * Both casts round to nearest even; products accumulate in fp32, in an order
 * fixed by (layout, m), so repeated calls give identical bits.
 * codes, params, x, y as for uq_gemv.
 * workspace : device memory owned by the caller, 256-byte aligned, of at
 *   least uq_gemm_workspace_size(layout, m) bytes (workspace_bytes says how
 *   many it has; fewer gives UQ_ERR_WORKSPACE, NULL UQ_ERR_NULL, misaligned
 *   UQ_ERR_ALIGN).  It must hold zeros before its first use with uq_gemm
 *   (allocate it zero-filled once); every call leaves it fit for the next
 *   one (the arrival counters it keeps in its first 64 KiB back at zero), so
 *   it is not cleared per call.  It holds bf16(x) for m > 64 and, for
 *   m <= 64, where the K dimension of a tile may be split over several
 *   workgroups, their partial tiles and arrival counters; the last
 *   workgroup of a tile adds the partial tiles in a fixed order, so results
 *   stay bitwise repeatable.  Calls that share a workspace must be ordered
 *   (e.g. issued to one stream); calls that may run concurrently need
 *   different workspaces.  Nothing else may write the workspace between
 *   calls.  A call may be captured into a HIP graph: it launches kernels
 *   only. */
uq_status uq_gemm(const uq_layout* layout, const void* codes, const void* params,
                  const uint16_t* x, float* y, int64_t m, void* workspace,
                  size_t workspace_bytes, void* stream);

/* uq_gemm for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the same product, kernels and results as uq_gemm, with the workspace taken
 * from a fixed device array of UQ_GEMM_NOALLOC_MAX_BYTES that the library
 * holds on each GPU it runs on until the process ends.  Calls whose
 * workspace (uq_gemm_workspace_size) would exceed that return
 * UQ_ERR_WORKSPACE before any HIP call.  Every call on a GPU shares that
 * GPU's array: calls that may overlap on one GPU (concurrent streams, or
 * threads) race and must not be made.  The first call on a device also
 * clears the array's arrival counters, by a kernel on `stream`.  Arguments
 * otherwise as for uq_gemm; allocates nothing. */
#define UQ_GEMM_NOALLOC_MAX_BYTES (32u << 20) /* 32 MiB per GPU */
uq_status uq_gemm_noalloc(const uq_layout* layout, const void* codes,
                          const void* params, const uint16_t* x, float* y,
                          int64_t m, void* stream);

/* Dequantize the whole matrix (the matching dequantizer of
 * Core Components > Quantization):  w[n][k] = w' exactly (bit for bit).
 *   w : device fp32 [n][k] row-major, 16-byte aligned, overwritten */
uq_status uq_dequant(const uq_layout* layout, const void* codes,
                     const void* params, float* w, void* stream);

/* ---- Dynamically quantized activations (Core Components > Quantized Model:
 * the quantized layers quantize their activations on the fly; the page names
 * no scheme, so this one is a reading). ----
 *
 * GEMV with int8 activations for the INT family (INT2/4/8 weights):
 *   per activation row m and weight group g, a = max |x[m][k]| over the group,
 *   q_x = clamp(rint(x * (127 / a)), -127, 127) with 127 / a and the product
 *   rounded to fp32 (ties to even; a = 0 gives q_x = 0), s_x = a / 127 (fp32);
 *   y[m][n] = sum_g s_x[m][g] * (s[n][g] * D + z[n][g] * Q),
 *   D = sum_{k in g} q_w[n][k] * q_x[m][k],  Q = sum_{k in g} q_x[m][k]
 * with D and Q exact integers and the scaling in fp32, for 1 <= m <= 8.
 * Arguments as for uq_gemv.  NF4 layouts return UQ_ERR_UNSUPPORTED (its
 * codebook values are not integers).  Allocates nothing. */
uq_status uq_gemv_a8(const uq_layout* layout, const void* codes,
                     const void* params, const uint16_t* x, float* y, int64_t m,
                     void* stream);

/* The activation quantization of uq_gemv_a8 on its own (test hook):
 *   x  : device fp16 [m][k] (uint16 bits), 16-byte aligned, k % group == 0, k % 16 == 0
 *   q  : device int8 [m][k], 16-byte aligned, overwritten with q_x
 *   sx : device fp32 [m][k / group], 4-byte aligned, overwritten with s_x
 * group in {16, 32, 64, 128}; 1 <= m <= 65536; 16 <= k <= 2^24. */
uq_status uq_quantize_activations(int32_t group, const uint16_t* x, int8_t* q,
                                  float* sx, int64_t m, int64_t k, void* stream);

/* ---- GGUF weight blocks (the "Ultra LLM Engine" page's Roadmap Ideas: Q4_0
 * and Q8_0 dequantizers; its Checkpoint Loading section: formats the loader
 * cannot decode are refused, not guessed).  The block layout is the public
 * GGUF one; the pages do not print it. ---- */
typedef enum uq_gguf_type {
  UQ_GGUF_Q4_0 = 2, /* GGUF tensor type ids */
  UQ_GGUF_Q8_0 = 8
} uq_gguf_type;

/* Re-lay GGUF Q4_0 / Q8_0 blocks of a weight matrix W[n][k] into this
 * library's INT layout, host call, exact:
 *   blocks : host, the tensor's data: n rows of k / 32 blocks, row-major;
 *            Q4_0 block = fp16 d (little-endian) + 16 bytes (byte j: weight j
 *            in the low nibble, weight j + 16 in the high), w = (nibble - 8) d;
 *            Q8_0 block = fp16 d + 32 int8 q, w = q d
 *   layout : written: Q4_0 -> {UQ_INT4, 32, n, k}, Q8_0 -> {UQ_INT8, 32, n, k}
 *   codes, params : host, uq_packed_size(layout) bytes, written
 * The result holds s = d and z = -8 d (Q4_0) or -128 d (Q8_0) per block and
 * codes nibble (Q4_0) or q + 128 (Q8_0), so uq_dequant returns every weight
 * exactly (as a number: a zero may change sign) and uq_gemv / uq_gemm /
 * uq_gemv_a8 serve the weights as any INT layout.  Errors: UQ_ERR_UNSUPPORTED
 * for another type; UQ_ERR_SHAPE unless n >= 1, k is a multiple of 32 and
 * k <= 2^24; UQ_ERR_RANGE if a scale is NaN or infinite or its zero point
 * exceeds fp16 (|d| >= 8192 for Q4_0, >= 512 for Q8_0).  All scales are
 * checked before anything is written. */
uq_status uq_import_gguf(int32_t gguf_type, const void* blocks, int64_t n,
                         int64_t k, uq_layout* layout, uint8_t* codes,
                         uint16_t* params);

/* The 16 NF4 codebook entries (fp32) the library uses; host call. */
uq_status uq_nf4_codebook(float out[16]);

/* ---- RMSNorm followed by RoPE (Core Components > Fused Kernels, third
 * bullet; the Architecture diagram's "RMSNorm + RoPE" step of each layer). ----
 *
 * Rotary table for uq_rmsnorm_rope, host call:
 *   cos[p][i] = fp32(cos(p * theta^(-2i/head_dim))), sin likewise, for
 *   0 <= p < max_pos, 0 <= i < head_dim/2; the angle is formed in fp64 and
 *   rounded once.  cos, sin: host fp32 [max_pos][head_dim/2], written.
 * UQ_ERR_SHAPE unless head_dim is even and >= 2, 1 <= max_pos <= 2^24 and
 * theta > 0 is finite. */
uq_status uq_rope_table(double theta, int32_t head_dim, int64_t max_pos,
                        float* cos, float* sin);

/* Fused RMSNorm + RoPE over vectors of head_dim values:
 *   u = x / sqrt(mean(x^2) + eps) * gamma           (over the head_dim values)
 *   y[i] = u[i] c - u[i+h] s,  y[i+h] = u[i+h] c + u[i] s,  i < h = head_dim/2,
 *   with c = cos[pos[t]][i], s = sin[pos[t]][i] for token t.
 *   x     : device fp16 [tokens][heads][head_dim] (uint16 bit patterns), 16-byte aligned
 *   y     : device fp16, same shape; may be x itself (in place)
 *   gamma : device fp32 [head_dim], 16-byte aligned
 *   pos   : device int32 [tokens], each in [0, max_pos)
 *   cos, sin : device fp32 [max_pos][head_dim/2] (e.g. from uq_rope_table), 16-byte aligned
 *   head_dim in {64, 128, 256, 512}; tokens >= 0 (0 launches nothing); heads >= 1;
 *   eps finite and >= 0.
 * Computed in fp32, rounded to fp16 (nearest even) once: within one fp16
 * spacing of the exact result, plus fp32 rounding at the vector's scale
 * (2^-18 of its largest output) where cancellation makes a value tiny.  A token whose position lies outside
 * [0, max_pos) gets NaN in every output value (the host cannot see device
 * positions; the kernel never reads outside the table). */
uq_status uq_rmsnorm_rope(const uint16_t* x, uint16_t* y, const float* gamma,
                          const int32_t* pos, const float* cos, const float* sin,
                          int64_t tokens, int32_t heads, int32_t head_dim,
                          int64_t max_pos, float eps, void* stream);

/* Measurement hook (not part of the product path): the streaming-read
 * ceiling of the decode GEMV, which reads each packed weight byte once
 * (Core Components > Fused Kernels, GEMV during single-token decode).
 * Reads every byte of [src, src + bytes) once with the GEMV's load pattern
 * (wave-wide 128-bit non-temporal loads, 1 KB per wave instruction,
 * `loads_in_flight` loads per lane before any is used), over `workgroups`
 * workgroups of 4 waves that each take an equal contiguous run of 1 KB
 * blocks; bytes = 0 launches a kernel that reads nothing.
 *   src  : device, 16-byte aligned; bytes a multiple of 1024
 *   sink : device uint32 [workgroups * 4], written with per-wave XORs of the data
 *   workgroups in 1 .. 2^20; loads_in_flight in {4, 8, 16, 32} */
uq_status uq_probe_read(const void* src, size_t bytes, int32_t workgroups,
                        int32_t loads_in_flight, uint32_t* sink, void* stream);

/* Static, NUL-terminated name of a status code ("UQ_OK", ...). */
const char* uq_status_str(uq_status status);

#ifdef __cplusplus
}
#endif

#endif /* UQ_H */
