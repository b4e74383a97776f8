// Host-side entry points of libuq under AddressSanitizer + UndefinedBehavior-
// Sanitizer (built by tests/test_sanitizers.py with g++, no HIP): the packer,
// the GGUF re-layout, the rotary table, the GEMM workspace size and the
// argument checks of the device entry points.
//
//   sanitize_driver pack   SCHEME GROUP N K W.f32 CODES.out PARAMS.out
//   sanitize_driver gguf   TYPE N K BLOCKS.bin CODES.out PARAMS.out
//   sanitize_driver rope   THETA HEAD_DIM MAX_POS COS.out SIN.out
//   sanitize_driver checks
//
// Output files hold the raw arrays; the Python side compares them with the
// oracle.  `checks` runs the error paths and exits non-zero on the first
// status that differs from the documented one.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "uq_internal.h"

namespace {

std::vector<unsigned char> read_file(const char* path) {
  std::vector<unsigned char> v;
  FILE* f = std::fopen(path, "rb");
  if (!f) return v;
  unsigned char buf[65536];
  size_t got;
  while ((got = std::fread(buf, 1, sizeof buf, f)) > 0) v.insert(v.end(), buf, buf + got);
  std::fclose(f);
  return v;
}

bool write_file(const char* path, const void* data, size_t bytes) {
  FILE* f = std::fopen(path, "wb");
  if (!f) return false;
  const bool ok = std::fwrite(data, 1, bytes, f) == bytes;
  return std::fclose(f) == 0 && ok;
}

int fail(const char* what, int got, int want) {
  std::fprintf(stderr, "check failed: %s: status %d, expected %d\n", what, got, want);
  return 1;
}

#define EXPECT(call, want)                              \
  do {                                                  \
    const int st_ = int(call);                          \
    if (st_ != int(want)) return fail(#call, st_, want); \
  } while (0)

int checks() {
  // layouts
  uq_layout bad_scheme = {9, 64, 4, 256}, bad_group = {UQ_INT4, 16, 4, 256}, bad_n = {UQ_INT4, 64, 0, 256},
            bad_k = {UQ_INT4, 64, 4, 96}, big_k = {UQ_INT4, 64, 4, (int64_t(1) << 24) + 64},
            big_n = {UQ_INT4, 64, int64_t(1) << 31, 256}, ok = {UQ_INT4, 64, 128, 256};
  size_t cb = 0, pb = 0;
  EXPECT(uq_packed_size(nullptr, &cb, &pb), UQ_ERR_NULL);
  EXPECT(uq_packed_size(&bad_scheme, &cb, &pb), UQ_ERR_UNSUPPORTED);
  EXPECT(uq_packed_size(&bad_group, &cb, &pb), UQ_ERR_UNSUPPORTED);
  EXPECT(uq_packed_size(&bad_n, &cb, &pb), UQ_ERR_SHAPE);
  EXPECT(uq_packed_size(&bad_k, &cb, &pb), UQ_ERR_SHAPE);
  EXPECT(uq_packed_size(&big_k, &cb, &pb), UQ_ERR_SHAPE);
  EXPECT(uq_packed_size(&big_n, &cb, &pb), UQ_ERR_SHAPE);
  EXPECT(uq_packed_size(&ok, nullptr, &pb), UQ_ERR_NULL);
  EXPECT(uq_packed_size(&ok, &cb, &pb), UQ_OK);
  if (cb != 128 * 128 || pb != 128 * 4 * 4) return fail("packed sizes", int(cb), 128 * 128);
  // the largest layout: sizes in 64 bits
  uq_layout huge = {UQ_INT4, 64, 0x7fffffff, int64_t(1) << 24};
  EXPECT(uq_packed_size(&huge, &cb, &pb), UQ_OK);
  if (cb != size_t(0x7fffffff) * (size_t(1) << 23)) return fail("huge code bytes", 0, 1);

  // packer errors (checked before anything is written)
  std::vector<float> w(2 * 64, 0.0f);
  std::vector<uint8_t> codes(64, 0xAB);
  std::vector<uint16_t> params(8, 0xABAB);
  uq_layout small = {UQ_INT4, 32, 2, 64};
  EXPECT(uq_pack_weights(&small, nullptr, codes.data(), params.data()), UQ_ERR_NULL);
  EXPECT(uq_pack_weights(&small, w.data(), nullptr, params.data()), UQ_ERR_NULL);
  for (float bad : {NAN, INFINITY, -INFINITY, 65505.0f, -70000.0f}) {
    w[77] = bad;
    EXPECT(uq_pack_weights(&small, w.data(), codes.data(), params.data()), UQ_ERR_RANGE);
    for (uint8_t c : codes)
      if (c != 0xAB) return fail("codes written before the range check", c, 0xAB);
  }
  w[77] = 0.5f;
  EXPECT(uq_pack_weights(&small, w.data(), codes.data(), params.data()), UQ_OK);

  // GEMM workspace: size and checks
  uq_layout g = {UQ_INT4, 128, 11008, 4096};
  size_t ws = 0;
  EXPECT(uq_gemm_workspace_size(&g, 0, &ws), UQ_ERR_SHAPE);
  EXPECT(uq_gemm_workspace_size(&g, UQ_GEMM_MAX_M + 1, &ws), UQ_ERR_SHAPE);
  EXPECT(uq_gemm_workspace_size(&g, 16, nullptr), UQ_ERR_NULL);
  for (int64_t m : {1, 16, 64, 65, 256, 4097, 65536}) {
    EXPECT(uq_gemm_workspace_size(&g, m, &ws), UQ_OK);
    void* fake = reinterpret_cast<void*>(uintptr_t(1) << 20);
    EXPECT(uq::check_gemm_workspace(&g, m, nullptr, ws), UQ_ERR_NULL);
    EXPECT(uq::check_gemm_workspace(&g, m, reinterpret_cast<char*>(fake) + 16, ws), UQ_ERR_ALIGN);
    EXPECT(uq::check_gemm_workspace(&g, m, fake, ws - 1), UQ_ERR_WORKSPACE);
    EXPECT(uq::check_gemm_workspace(&g, m, fake, ws), UQ_OK);
  }

  // product / dequant / quantizer / rmsnorm-rope argument checks
  const void* A = reinterpret_cast<const void*>(uintptr_t(1) << 20);
  const char* Ab = static_cast<const char*>(A);
  EXPECT(uq::check_product(nullptr, A, A, A, A, 1, 8), UQ_ERR_NULL);
  EXPECT(uq::check_product(&ok, nullptr, A, A, A, 1, 8), UQ_ERR_NULL);
  EXPECT(uq::check_product(&ok, A, A, A, A, 0, 8), UQ_ERR_SHAPE);
  EXPECT(uq::check_product(&ok, A, A, A, A, 9, 8), UQ_ERR_SHAPE);
  EXPECT(uq::check_product(&ok, Ab + 4, A, A, A, 1, 8), UQ_ERR_ALIGN);
  EXPECT(uq::check_product(&ok, A, A, Ab + 2, A, 1, 8), UQ_ERR_ALIGN);
  EXPECT(uq::check_product(&ok, A, A, A, A, 8, 8), UQ_OK);
  EXPECT(uq::check_dequant(&ok, A, A, Ab + 8), UQ_ERR_ALIGN);
  EXPECT(uq::check_quantize_activations(48, A, A, A, 1, 256), UQ_ERR_UNSUPPORTED);
  EXPECT(uq::check_quantize_activations(64, A, A, A, 1, 96), UQ_ERR_SHAPE);
  EXPECT(uq::check_quantize_activations(64, A, A, Ab + 2, 1, 256), UQ_ERR_ALIGN);
  EXPECT(uq::check_rmsnorm_rope(A, A, A, A, A, A, 4, 2, 96, 64, 1e-6f), UQ_ERR_UNSUPPORTED);
  EXPECT(uq::check_rmsnorm_rope(A, A, A, A, A, A, -1, 2, 128, 64, 1e-6f), UQ_ERR_SHAPE);
  EXPECT(uq::check_rmsnorm_rope(A, A, A, A, A, A, 4, 2, 128, 64, NAN), UQ_ERR_RANGE);
  EXPECT(uq::check_rmsnorm_rope(A, A, A, A, A, A, int64_t(1) << 40, 2, 128, 64, 1e-6f), UQ_ERR_SHAPE);
  EXPECT(uq::check_probe_read(A, 1000, 4, 8, A), UQ_ERR_SHAPE);
  EXPECT(uq::check_probe_read(A, 1024, 4, 3, A), UQ_ERR_UNSUPPORTED);

  // GGUF errors (all scales checked before anything is written)
  std::vector<uint8_t> blocks(3 * 4 * 18, 0);
  uq_layout lay;
  std::vector<uint8_t> gc(3 * 128, 0xAB);
  std::vector<uint16_t> gp(3 * 4 * 2, 0xABAB);
  EXPECT(uq_import_gguf(3, blocks.data(), 3, 128, &lay, gc.data(), gp.data()), UQ_ERR_UNSUPPORTED);
  EXPECT(uq_import_gguf(UQ_GGUF_Q4_0, blocks.data(), 3, 48, &lay, gc.data(), gp.data()), UQ_ERR_SHAPE);
  EXPECT(uq_import_gguf(UQ_GGUF_Q4_0, nullptr, 3, 128, &lay, gc.data(), gp.data()), UQ_ERR_NULL);
  blocks[blocks.size() - 18] = 0x00;  // last block's d = +inf (0x7C00)
  blocks[blocks.size() - 17] = 0x7C;
  EXPECT(uq_import_gguf(UQ_GGUF_Q4_0, blocks.data(), 3, 128, &lay, gc.data(), gp.data()), UQ_ERR_RANGE);
  for (uint8_t c : gc)
    if (c != 0xAB) return fail("GGUF codes written before the scale check", c, 0xAB);

  // rotary table errors
  std::vector<float> cs(64), sn(64);
  EXPECT(uq_rope_table(1e4, 7, 4, cs.data(), sn.data()), UQ_ERR_SHAPE);
  EXPECT(uq_rope_table(0.0, 8, 4, cs.data(), sn.data()), UQ_ERR_SHAPE);
  EXPECT(uq_rope_table(NAN, 8, 4, cs.data(), sn.data()), UQ_ERR_SHAPE);
  EXPECT(uq_rope_table(1e4, 8, 4, nullptr, sn.data()), UQ_ERR_NULL);

  // constants
  float cb16[16];
  EXPECT(uq_nf4_codebook(cb16), UQ_OK);
  EXPECT(uq_nf4_codebook(nullptr), UQ_ERR_NULL);
  for (int s = 0; s <= 7; ++s)
    if (!uq_status_str(uq_status(s))) return fail("status string", s, 0);
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc >= 2 && std::strcmp(argv[1], "checks") == 0) return checks();
  if (argc == 9 && std::strcmp(argv[1], "pack") == 0) {
    uq_layout L = {std::atoi(argv[2]), std::atoi(argv[3]), std::atoll(argv[4]), std::atoll(argv[5])};
    size_t cb = 0, pb = 0;
    if (uq_packed_size(&L, &cb, &pb) != UQ_OK) return 2;
    const std::vector<unsigned char> w = read_file(argv[6]);
    if (w.size() != size_t(L.n) * size_t(L.k) * 4) return 3;
    std::vector<float> wf(w.size() / 4);
    std::memcpy(wf.data(), w.data(), w.size());
    std::vector<uint8_t> codes(cb);
    std::vector<uint16_t> params(pb / 2);
    const uq_status st = uq_pack_weights(&L, wf.data(), codes.data(), params.data());
    if (st != UQ_OK) return 10 + int(st);
    return write_file(argv[7], codes.data(), cb) && write_file(argv[8], params.data(), pb) ? 0 : 4;
  }
  if (argc == 8 && std::strcmp(argv[1], "gguf") == 0) {
    const int type = std::atoi(argv[2]);
    const int64_t n = std::atoll(argv[3]), k = std::atoll(argv[4]);
    const std::vector<unsigned char> blocks = read_file(argv[5]);
    const size_t bb = type == UQ_GGUF_Q4_0 ? 18 : 34;
    if (blocks.size() != size_t(n) * size_t(k / 32) * bb) return 3;
    std::vector<uint8_t> codes(size_t(n) * size_t(k));
    std::vector<uint16_t> params(size_t(n) * size_t(k / 32) * 2);
    uq_layout L;
    const uq_status st = uq_import_gguf(type, blocks.data(), n, k, &L, codes.data(), params.data());
    if (st != UQ_OK) return 10 + int(st);
    size_t cb = 0, pb = 0;
    if (uq_packed_size(&L, &cb, &pb) != UQ_OK) return 2;
    return write_file(argv[6], codes.data(), cb) && write_file(argv[7], params.data(), pb) ? 0 : 4;
  }
  if (argc == 7 && std::strcmp(argv[1], "rope") == 0) {
    const double theta = std::atof(argv[2]);
    const int d = std::atoi(argv[3]);
    const int64_t p = std::atoll(argv[4]);
    std::vector<float> c(size_t(p) * size_t(d / 2)), s(c.size());
    const uq_status st = uq_rope_table(theta, d, p, c.data(), s.data());
    if (st != UQ_OK) return 10 + int(st);
    return write_file(argv[5], c.data(), c.size() * 4) && write_file(argv[6], s.data(), s.size() * 4) ? 0 : 4;
  }
  std::fprintf(stderr, "usage: see the header of sanitize_driver.cpp\n");
  return 64;
}
