// Host-side driver for the AddressSanitizer pass over libqgemm's argument
// checks (built and run by test_host_asan.py; no GPU needed).  Every call
// below is rejected or finishes on the host before anything is launched, so
// only the library's host code runs; the sanitizer reports any bad memory
// access in that code.  Exits 0 when every status is the expected one.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "qgemm.h"

namespace {

int failures = 0;

void expect(const char* what, long long got, long long want) {
  if (got != want) {
    std::printf("FAIL %s: got %lld, want %lld\n", what, got, want);
    ++failures;
  }
}

void* P(unsigned long long v) { return reinterpret_cast<void*>(v); }

}  // namespace

int main() {
  void* good = P(0x10000);   // 16-byte aligned, never dereferenced by these calls
  void* odd = P(0x10008);
  void* s = nullptr;

  // status strings: every code, and an unknown one
  for (int st = 0; st >= -7; --st) {
    const char* t = qgemm_status_string(st);
    expect("status string present", t != nullptr && std::strlen(t) > 0, 1);
  }
  expect("unknown status", std::strcmp(qgemm_status_string(999), "unknown status"), 0);

  // sizes
  expect("prepack bytes w4", qgemm_prepack_bytes(QGEMM_W4A16, 1024, 1024), 1024 * 1024 / 2);
  expect("prepack bytes odd K", qgemm_prepack_bytes(QGEMM_W4A16, 3, 5), QGEMM_ERR_SHAPE);
  expect("prepack bytes format", qgemm_prepack_bytes(9, 32, 32), QGEMM_ERR_FORMAT);
  expect("grouped bytes", qgemm_prepack_grouped_bytes(QGEMM_W4A16_GROUPED, 4096, 4096, 48),
         QGEMM_ERR_SHAPE);
  expect("act ws fp8", qgemm_act_workspace_bytes(QGEMM_FP8, 16, 8192), 16 * 8192 + 16 + 1024);
  expect("act ws format", qgemm_act_workspace_bytes(QGEMM_W4A16, 16, 64), QGEMM_ERR_FORMAT);

  // argument errors of every GEMM family
  expect("w8 null", qgemm_w8a16(nullptr, good, good, good, 4, 4, 32, s), QGEMM_ERR_NULL);
  expect("w4 shape", qgemm_w4a16(good, good, good, good, 4, 4, 31, s), QGEMM_ERR_SHAPE);
  expect("w4 align", qgemm_w4a16(good, odd, good, good, 4, 4, 32, s), QGEMM_ERR_ALIGN);
  expect("w8 empty", qgemm_w8a16(good, good, good, good, 0, 4, 32, s), QGEMM_OK);
  expect("w8 overflow", qgemm_w8a16(good, good, good, good, 1 << 20, 1 << 20, 64, s),
         QGEMM_ERR_SHAPE);
  expect("mx null", qgemm_mxfp4(good, good, nullptr, good, 4, 4, 32, s), QGEMM_ERR_NULL);
  expect("mx shape", qgemm_mxfp4(good, good, good, good, 4, 4, 48, s), QGEMM_ERR_SHAPE);
  expect("fp8 scale align",
         qgemm_fp8(good, good, static_cast<const float*>(P(0x10002)), static_cast<float*>(good),
                   good, 4, 4, 32, s),
         QGEMM_ERR_ALIGN);
  expect("nvfp4 null", qgemm_nvfp4(good, good, nullptr, good, 4, 16, 64, s), QGEMM_ERR_NULL);
  expect("grouped shape", qgemm_w4a16_grouped(good, good, good, 4, 16, 120, 128, s),
         QGEMM_ERR_SHAPE);
  expect("prepack format", qgemm_prepack(9, good, nullptr, good, 32, 32, s), QGEMM_ERR_FORMAT);
  expect("prepack grouped n", qgemm_prepack_grouped(QGEMM_W4A16_GROUPED, good, good, nullptr, 128,
                                                    0, good, 128, 16, s),
         QGEMM_ERR_SHAPE);
  expect("quantize mx shape",
         qgemm_quantize_mxfp4(static_cast<const float*>(good), 4, 48,
                              static_cast<uint8_t*>(good), static_cast<uint8_t*>(good), s),
         QGEMM_ERR_SHAPE);
  expect("quantize fp8 null",
         qgemm_quantize_fp8(static_cast<const float*>(good), 16, static_cast<uint8_t*>(good),
                            nullptr, s),
         QGEMM_ERR_NULL);
  expect("mx act null", qgemm_mxfp4_act(static_cast<const float*>(good), good, good, nullptr, 4,
                                        16, 64, s),
         QGEMM_ERR_NULL);
  expect("fp8 act shape",
         qgemm_fp8_act(static_cast<const float*>(good), good, static_cast<const float*>(good),
                       good, good, 4, 16, 40, s),
         QGEMM_ERR_SHAPE);

  // the architecture check, with the architecture name injected
  setenv("QGEMM_ARCH_OVERRIDE", "gfx942", 1);
  expect("arch w8", qgemm_w8a16(good, good, good, good, 4, 16, 32, s), QGEMM_ERR_ARCH);
  expect("arch fp8 act",
         qgemm_fp8_act(static_cast<const float*>(good), good, static_cast<const float*>(good),
                       good, good, 4, 16, 64, s),
         QGEMM_ERR_ARCH);
  unsetenv("QGEMM_ARCH_OVERRIDE");

  // the dispatch query (host-only)
  expect("dispatch w8a16 decode", qgemm_dispatch_kernel(QGEMM_W8A16, 16, 11008, 4096, 0),
         QGEMM_KERNEL_SMALL_M);
  expect("dispatch w4a16 square", qgemm_dispatch_kernel(QGEMM_W4A16, 4096, 4096, 4096, 0),
         QGEMM_KERNEL_WEIGHT_ONLY_256);
  expect("dispatch mxfp4 square", qgemm_dispatch_kernel(QGEMM_MXFP4, 8192, 8192, 8192, 0),
         QGEMM_KERNEL_MXFP4_256);
  expect("dispatch empty", qgemm_dispatch_kernel(QGEMM_FP8, 0, 64, 64, 0), QGEMM_KERNEL_NONE);
  expect("dispatch format", qgemm_dispatch_kernel(99, 4, 4, 32, 0), QGEMM_ERR_FORMAT);
  expect("dispatch shape", qgemm_dispatch_kernel(QGEMM_MXFP4, 4, 4, 40, 0), QGEMM_ERR_SHAPE);
  expect("dispatch group", qgemm_dispatch_kernel(QGEMM_W4A16_GROUPED, 4, 4, 64, 48),
         QGEMM_ERR_SHAPE);

  std::printf("%s (%d failures)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
