// abi_host_driver.cpp -- drives the host-side validation of every C-ABI entry
// point (include/ssmdec.h) with arguments that must be rejected, for a build
// of ssmd_api.hip with host-side AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_sanitizers.py). Every call here is
// refused before any HIP call (pointers are fake and never dereferenced), and
// the process hides every GPU from itself before the first HIP call, so
// nothing can be launched even on a machine with a GPU.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ssmdec.h"

static int fails = 0;
static void expect(int got, int want, const char* what) {
  const char* msg = ssmd_last_error();
  if (got != want || (want != SSMD_OK && (!msg || !msg[0]))) {
    fprintf(stderr, "%s: got %d want %d (%s)\n", what, got, want, msg ? msg : "(null)");
    ++fails;
  }
}

#define P(x) reinterpret_cast<void*>(uintptr_t(x))
#define FP(x) reinterpret_cast<float*>(uintptr_t(x))
#define IP(x) reinterpret_cast<int32_t*>(uintptr_t(x))

static int gdn(const void* qkv, int64_t stride, void* state, const int32_t* idx, int B, int H, int HV, int K, int V,
               int act, int odt, int nact) {
  return gdn_decode_step(qkv, stride, P(0x20000), P(0x30000), FP(0x40000), FP(0x50000), (float*)state, 16, idx,
                         P(0x80000), B, H, HV, K, V, act, odt, 0.088f, 1, 1e-6f, nullptr, nullptr, 1e-5f, nact,
                         nullptr);
}

int main() {
  setenv("HIP_VISIBLE_DEVICES", "-1", 1);
  setenv("ROCR_VISIBLE_DEVICES", "-1", 1);
  const void* q = P(0x10000);
  void* st = P(0x60000);
  const int32_t* ix = IP(0x70000);
  // packed step
  expect(gdn(nullptr, 8192, st, ix, 16, 16, 32, 128, 128, 1, 1, 0), SSMD_ERR_NULL_ARG, "gdn null qkv");
  expect(gdn(q, 8192, nullptr, ix, 16, 16, 32, 128, 128, 1, 1, 0), SSMD_ERR_NULL_ARG, "gdn null state");
  expect(gdn(q, 8192, st, nullptr, 16, 16, 32, 128, 128, 1, 1, 0), SSMD_ERR_NULL_ARG, "gdn null idx");
  expect(gdn(q, 8192, st, ix, 16, 16, 24, 128, 128, 1, 1, 0), SSMD_ERR_BAD_SHAPE, "gdn HV % H");
  expect(gdn(q, 8192, st, ix, 16, 0, 32, 128, 128, 1, 1, 0), SSMD_ERR_BAD_SHAPE, "gdn H = 0");
  expect(gdn(q, 8192, st, ix, 16, 16, 32, 48, 128, 1, 1, 0), SSMD_ERR_UNSUPPORTED, "gdn K = 48");
  expect(gdn(q, 8192, st, ix, 16, 16, 32, 128, 0, 1, 1, 0), SSMD_ERR_BAD_SHAPE, "gdn V = 0");
  expect(gdn(q, 8192, st, ix, 16, 16, 32, 128, 2048, 1, 1, 0), SSMD_ERR_BAD_SHAPE, "gdn V = 2048");
  expect(gdn(q, 8192, st, ix, -1, 16, 32, 128, 128, 1, 1, 0), SSMD_ERR_BAD_SHAPE, "gdn B < 0");
  expect(gdn(q, 8192, st, ix, 16, 16, 32, 128, 128, 7, 1, 0), SSMD_ERR_BAD_DTYPE, "gdn act dtype");
  expect(gdn(q, 8192, st, ix, 16, 16, 32, 128, 128, 1, -1, 0), SSMD_ERR_BAD_DTYPE, "gdn out dtype");
  expect(gdn(q, 8192, st, ix, 16, 16, 32, 128, 128, 1, 1, 3), SSMD_ERR_BAD_DTYPE, "gdn norm act");
  expect(gdn(q, 8191, st, ix, 16, 16, 32, 128, 128, 1, 1, 0), SSMD_ERR_BAD_SHAPE, "gdn row stride");
  expect(gdn(q, 8192, P(0x60004), ix, 16, 16, 32, 128, 128, 1, 1, 0), SSMD_ERR_BAD_SHAPE, "gdn state alignment");
  expect(gdn(nullptr, 8192, nullptr, nullptr, 0, 16, 32, 128, 128, 1, 1, 0), SSMD_OK, "gdn B = 0");
  // 16-bit state
  expect(gdn_decode_step_state16(q, 8192, P(2), P(3), FP(4), FP(8), st, SSMD_F32, 16, ix, P(9), 16, 16, 32, 128, 128,
                                 1, 1, 0.088f, 1, 1e-6f, nullptr, nullptr, 1e-5f, 0, nullptr),
         SSMD_ERR_BAD_DTYPE, "state16 fp32 pool");
  // buffered
  for (int L : {0, 65})
    expect(gdn_decode_step_buffered(q, 8192, P(2), P(3), FP(4), FP(8), FP(0x60000), 16, ix, P(9), 4, 16, 32, 128,
                                    128, 1, 1, 0.088f, 1, 1e-6f, nullptr, nullptr, 1e-5f, 0, P(0x90000), P(0xB0000),
                                    FP(0xC0000), IP(0xA0000), L, nullptr),
           SSMD_ERR_BAD_SHAPE, "buffered L");
  expect(gdn_decode_step_buffered(q, 8192, P(2), P(3), FP(4), FP(8), FP(0x60000), 16, ix, P(9), 4, 16, 32, 128, 128,
                                  1, 1, 0.088f, 1, 1e-6f, nullptr, nullptr, 1e-5f, 0, nullptr, P(0xB0000),
                                  FP(0xC0000), IP(0xA0000), 8, nullptr),
         SSMD_ERR_NULL_ARG, "buffered null ring");
  // multi-token, chunked prefill, its static-workspace variant
  expect(gdn_fused_recurrent(q, 8192, P(2), P(3), FP(4), FP(8), FP(0x60000), 16, ix, nullptr, P(9), 4, -3, 16, 32,
                             128, 128, 1, 1, 0.088f, 1, 1e-6f, nullptr, nullptr, 1e-5f, 0, nullptr),
         SSMD_ERR_BAD_SHAPE, "multi T < 0");
  expect(gdn_chunk_prefill(q, 8192, P(2), P(3), FP(4), FP(8), FP(0x60000), 16, ix, nullptr, P(9), 1, 128, 16, 32,
                           128, 128, 1, 1, 0.088f, 1, 1e-6f, nullptr, nullptr, 1e-5f, 0, nullptr, 0, nullptr),
         SSMD_ERR_BAD_SHAPE, "chunk no workspace");
  expect(gdn_chunk_prefill(q, 8192, P(2), P(3), FP(4), FP(8), FP(0x60000), 16, ix, nullptr, P(9), 1, 128, 16, 32,
                           32, 128, 1, 1, 0.088f, 1, 1e-6f, nullptr, nullptr, 1e-5f, 0, P(0x100000), 1 << 30, nullptr),
         SSMD_ERR_UNSUPPORTED, "chunk K = 32");
  expect(gdn_chunk_prefill_noalloc(q, 2176, P(2), P(3), FP(4), FP(8), FP(0x60000), 4, ix, nullptr, P(9), 1, 8192, 1,
                                   32, 64, 64, 1, 0, 0.125f, 1, 1e-6f, nullptr, nullptr, 1e-5f, 0, nullptr),
         SSMD_ERR_BAD_SHAPE, "chunk static workspace too small");
  expect(gdn_chunk_workspace_bytes(-1, 1, 1, 64, 64, 0) < 0 ? SSMD_ERR_BAD_SHAPE : SSMD_OK, SSMD_ERR_BAD_SHAPE,
         "chunk workspace bytes");
  // conv-fused GDN
  expect(gdn_decode_step_conv(q, 8192, FP(2), nullptr, P(3), 8192 * 3, 3, 1, 9, P(4), P(5), FP(6), FP(8),
                              FP(0x60000), 16, ix, P(9), 4, 16, 32, 128, 128, 1, 1, 0.088f, 1, 1e-6f, nullptr,
                              nullptr, 1e-5f, 0, nullptr),
         SSMD_ERR_BAD_SHAPE, "conv width 9");
  // KDA
  auto kda = [&](int T, int D, int W, const float* A_log, const float* dt_bias, const void* x) {
    return kda_decode_step(x, FP(0x20000), nullptr, P(0x30000), 216 * 128 * 3, 1, 36864, P(0x40000), P(0x50000),
                           A_log, dt_bias, -5.f, FP(0x60000), 72, IP(0x70000), P(0x80000), P(0x90000), nullptr, 1e-5f,
                           T, 96, D, W, 1, 1, 0.088f, 1, 1e-6f, nullptr);
  };
  expect(kda(64, 96, 4, nullptr, nullptr, q), SSMD_ERR_UNSUPPORTED, "kda D = 96");
  expect(kda(64, 128, 1, nullptr, nullptr, q), SSMD_ERR_BAD_SHAPE, "kda W = 1");
  expect(kda(64, 128, 4, nullptr, nullptr, nullptr), SSMD_ERR_NULL_ARG, "kda null x");
  expect(kda(64, 128, 4, FP(0xA0000), nullptr, q), SSMD_ERR_UNSUPPORTED, "kda A_log refused");
  expect(kda(0, 128, 4, nullptr, FP(0xB0000), q), SSMD_ERR_UNSUPPORTED, "kda dt_bias refused");
  // Mamba-1
  expect(mamba_decode_step(q, P(2), FP(4), P(5), P(6), nullptr, nullptr, FP(0x60000), 8, ix, P(9), 8, 1536, 48, 1, 1,
                           nullptr),
         SSMD_ERR_UNSUPPORTED, "mamba N = 48");
  expect(mamba_scan(q, P(2), FP(4), P(5), P(6), nullptr, nullptr, FP(0x60000), 8, ix, nullptr, 0, P(9), nullptr, -16,
                    8, 64, 1536, 16, 1, 1, nullptr),
         SSMD_ERR_BAD_SHAPE, "scan workspace < 0");
  expect(mamba_scan_workspace_bytes(-1, 1, 1, 16) < 0 ? SSMD_ERR_BAD_SHAPE : SSMD_OK, SSMD_ERR_BAD_SHAPE,
         "scan workspace bytes");
  // measurement aids
  expect(ssmd_stream_copy(nullptr, P(0x1000), 64, nullptr), SSMD_ERR_NULL_ARG, "copy null");
  expect(ssmd_stream_copy(P(0x1000), P(0x2000), 17, nullptr), SSMD_ERR_BAD_SHAPE, "copy size");
  expect(ssmd_check_slot_indices(ix, 70000, 8, 0, IP(0x3000), nullptr), SSMD_ERR_BAD_SHAPE, "check B");
  expect(ssmd_check_slot_indices(ix, 8, 8, 0, nullptr, nullptr), SSMD_ERR_NULL_ARG, "check null count");
  if (fails) {
    fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  printf("ABI_HOST_DRIVER_OK\n");
  return 0;
}
