// Calls every entry point of the C ABI (include/qmv.h) with arguments that
// host-side validation must refuse before any HIP call, plus the workspace
// sizing queries, so that a library whose host code is built with
// AddressSanitizer and UndefinedBehaviorSanitizer runs its validation paths
// (no GPU is touched).  Also checks that the error message is per thread.
// Prints "ok" and exits 0 when every call returns the expected code.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>

#include "qmv.h"

static int failures = 0;

static void expect(int rc, int want, const char *what) {
  if (rc != want) {
    std::printf("FAIL %s: rc=%d want=%d (%s)\n", what, rc, want, qmv_last_error());
    failures++;
  } else if (want != QMV_OK && std::strlen(qmv_last_error()) == 0) {
    std::printf("FAIL %s: no error message\n", what);
    failures++;
  }
}

int main() {
  // never dereferenced: every call below is refused before any access
  auto *x = reinterpret_cast<const uint16_t *>(0x10000);
  auto *w = reinterpret_cast<const uint32_t *>(0x20000);
  auto *s = reinterpret_cast<const uint16_t *>(0x30000);
  auto *b = reinterpret_cast<const uint16_t *>(0x40000);
  void *y = reinterpret_cast<void *>(0x50000);
  auto *xm = reinterpret_cast<const uint16_t *>(0x10002);   // not 16-byte aligned

  expect(qmv(x, w, s, b, y, 1, 16, 64, 64, 7, 1, 0, nullptr), QMV_EINVAL, "qmv bits=7");
  expect(qmv(x, w, s, b, y, 1, 16, 96, 64, 4, 1, 0, nullptr), QMV_EINVAL, "qmv K % g");
  expect(qmv(x, w, s, b, y, 1, 16, 64, 48, 4, 1, 0, nullptr), QMV_EINVAL, "qmv g=48");
  expect(qmv(x, w, s, b, y, 0, 16, 64, 64, 4, 1, 0, nullptr), QMV_EINVAL, "qmv M=0");
  expect(qmv(x, w, s, b, y, 1, 0, 64, 64, 4, 1, 0, nullptr), QMV_EINVAL, "qmv N=0");
  expect(qmv(x, w, s, b, y, 1, 16, 64, 64, 4, 2, 0, nullptr), QMV_EINVAL, "qmv transpose=2");
  expect(qmv(x, w, s, b, y, 1, 16, 64, 64, 4, 1, 9, nullptr), QMV_EINVAL, "qmv out_dtype=9");
  expect(qmv(nullptr, w, s, b, y, 1, 16, 64, 64, 4, 1, 0, nullptr), QMV_EINVAL, "qmv x=NULL");
  expect(qmv(xm, w, s, b, y, 1, 16, 64, 64, 4, 1, 0, nullptr), QMV_EINVAL, "qmv x misaligned");
  expect(qmv(x, w, s, b, y, 1, 100, 64, 64, 4, 0, 0, nullptr), QMV_EINVAL, "qmv transpose=0 N % g");

  size_t n = 1;
  expect(qmv_workspace_bytes(1, 4096, 4096, 64, 4, 1, &n), QMV_OK, "ws matvec");
  if (n != 0) { std::printf("FAIL ws matvec: %zu\n", n); failures++; }
  expect(qmv_workspace_bytes(1, 4096, 4096, 64, 4, 0, &n), QMV_OK, "ws qvm");
  if (n == 0 || n % (4 * 4096) != 0) { std::printf("FAIL ws qvm: %zu\n", n); failures++; }
  expect(qmv_workspace_bytes(64, 4096, 4096, 64, 4, 1, &n), QMV_OK, "ws qmm");
  if (n == 0 || n % (4 * 4096) != 0) { std::printf("FAIL ws qmm: %zu\n", n); failures++; }
  expect(qmv_workspace_bytes(1, 16, 96, 64, 4, 1, &n), QMV_EINVAL, "ws K % g");
  expect(qmv_workspace_bytes(1, 16, 64, 64, 4, 1, nullptr), QMV_EINVAL, "ws bytes=NULL");

  size_t need = 0;
  qmv_workspace_bytes(1, 4096, 4096, 64, 4, 0, &need);
  expect(qmv_with_workspace(x, w, s, b, y, 1, 4096, 4096, 64, 4, 0, 0, reinterpret_cast<void *>(0x60000),
                            need - 16, nullptr), QMV_EINVAL, "with_workspace too small");
  expect(qmv_with_workspace(x, w, s, b, y, 1, 4096, 4096, 64, 4, 0, 0, reinterpret_cast<void *>(0x60008),
                            need, nullptr), QMV_EINVAL, "with_workspace misaligned");
  expect(qmv_noalloc(x, w, s, b, y, 3, 65536, 65536, 64, 4, 0, 0, nullptr), QMV_EINVAL, "noalloc too large");
  expect(qmv_noalloc(x, w, s, b, y, 1, 16, 64, 64, 3, 1, 5, nullptr), QMV_EINVAL, "noalloc out_dtype");

  auto *g16 = reinterpret_cast<uint16_t *>(0x70000);
  expect(qmv_gate_up(x, w, s, b, w, s, b, g16, g16, 16, 64, 64, 1, nullptr), QMV_EINVAL, "gate_up bits=1");
  expect(qmv_gate_up(x, w, s, b, nullptr, s, b, g16, g16, 16, 64, 64, 4, nullptr), QMV_EINVAL,
         "gate_up wu=NULL");
  expect(qmv_silu_gate_resid(x, x, x, w, s, b, y, 16, 64, 64, 4, 7, nullptr), QMV_EINVAL, "silu out_dtype");
  expect(qmv_silu_gate_resid(x, nullptr, x, w, s, b, y, 16, 64, 64, 4, 0, nullptr), QMV_EINVAL, "silu up=NULL");

  auto *idx = reinterpret_cast<const uint32_t *>(0x80000);
  expect(gather_qmv(x, 2, w, s, b, 4, idx, nullptr, 8, y, 1, 16, 64, 64, 4, 1, 0, 0, nullptr), QMV_EINVAL,
         "gather one index NULL");
  expect(gather_qmv(x, 2, w, s, b, 4, idx, idx, 8, y, 1, 16, 64, 64, 4, 0, 0, 0, nullptr), QMV_EUNSUPPORTED,
         "gather transpose=0");
  expect(gather_qmv(x, 2, w, s, b, 4, idx, idx, 8, y, 1, 16, 64, 64, 9, 1, 0, 0, nullptr), QMV_EINVAL,
         "gather bits=9");
  expect(qmv_dequantize(w, s, b, y, 16, 96, 64, 4, 0, nullptr), QMV_EINVAL, "dequantize K % g");
  expect(qmv_dequantize(w, s, b, y, 16, 64, 64, 4, 3, nullptr), QMV_EINVAL, "dequantize out_dtype");
  expect(qmv_unpack_codes(w, 16, 48, 4, reinterpret_cast<uint8_t *>(0x90000), nullptr), QMV_EINVAL,
         "unpack K % 32");
  expect(qmv_pack(reinterpret_cast<const float *>(0xA0000), 16, 64, 64, 5, nullptr, g16, g16, nullptr),
         QMV_EINVAL, "pack w_q=NULL");
  expect(qmv_pack(reinterpret_cast<const float *>(0xA0004), 16, 64, 64, 4, reinterpret_cast<uint32_t *>(0xB0000),
                  g16, g16, nullptr), QMV_EINVAL, "pack w misaligned");

  // the message belongs to the thread that failed
  qmv(x, w, s, b, y, 1, 16, 64, 64, 7, 1, 0, nullptr);
  const std::string mine = qmv_last_error();
  std::string theirs;
  std::thread t([&] {
    qmv(x, w, s, b, y, 1, 16, 96, 64, 4, 1, 0, nullptr);
    theirs = qmv_last_error();
  });
  t.join();
  if (mine == theirs || mine != qmv_last_error()) {
    std::printf("FAIL per-thread message: '%s' / '%s'\n", mine.c_str(), theirs.c_str());
    failures++;
  }
  if (failures) {
    std::printf("%d failures\n", failures);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
