// Host sanitizer driver for the C ABI's validation layer (efla_api.hip built
// for the host with AddressSanitizer and UndefinedBehaviorSanitizer; CPU
// only, test infrastructure). The kernels' launch entry points are replaced
// by stubs that only count calls, so every public function runs its whole
// host path with no GPU: valid calls must reach exactly one launch and
// return EFLA_OK, invalid ones must return their error code with no launch.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include "efla.h"

static int launches = 0;
static size_t fwd_ws = 0;   // workspace the stubbed query reports for the forward
static size_t bwd_ws = 64;  // ... and for the backward

hipError_t efla_internal_launch_chunked(const void*, const void*, const void*, const void*, const float*,
                                        void*, float*, void*, int, int, int, int, int, int, hipStream_t) {
  ++launches;
  return hipSuccess;
}
size_t efla_internal_chunked_workspace_bytes(int, int, int, int, int) { return fwd_ws; }
hipError_t efla_internal_launch_decode(const void*, const void*, const void*, const void*, const float*, float*,
                                       void*, int, int, int, int, hipStream_t) {
  ++launches;
  return hipSuccess;
}
hipError_t efla_internal_launch_chunked_gated(const void*, const void*, const void*, const void*, const float*,
                                              const float*, void*, float*, int, int, int, int, int, int,
                                              hipStream_t) {
  ++launches;
  return hipSuccess;
}
size_t efla_internal_bwd_workspace_bytes(int, int, int, int, int) { return bwd_ws; }
hipError_t efla_internal_launch_bwd(const void*, const void*, const void*, const void*, const float*,
                                    const void*, const float*, void*, void*, void*, void*, float*, void*, int,
                                    int, int, int, int, int, int, hipStream_t) {
  ++launches;
  return hipSuccess;
}
hipError_t efla_internal_launch_fwd_save(const void*, const void*, const void*, const void*, const float*,
                                         void*, float*, void*, int, int, int, int, int, int, hipStream_t) {
  ++launches;
  return hipSuccess;
}

static int fails = 0;
static void expect(const char* what, int got, int want, int want_launches) {
  if (got != want || launches != want_launches) {
    printf("FAIL %s: status %d (want %d), launches %d (want %d)\n", what, got, want, launches,
           want_launches);
    ++fails;
  }
  launches = 0;
}

int main() {
  alignas(16) static char mem[1 << 12];
  void* P = mem;
  void* M = mem + 2;  // misaligned
  float* S = (float*)mem;
  const efla_coef X = EFLA_COEF_EXACT;
  const efla_dtype BF = EFLA_DTYPE_BF16, F32 = EFLA_DTYPE_F32;

  expect("fwd ok", efla_fwd_chunked(P, P, P, P, S, P, S, nullptr, 0, 2, 3, 100, 64, 64, 64, X, BF, nullptr),
         EFLA_OK, 1);
  expect("fwd null", efla_fwd_chunked(nullptr, P, P, P, S, P, S, nullptr, 0, 2, 3, 100, 64, 64, 64, X, BF,
                                      nullptr), EFLA_ERR_NULL_POINTER, 0);
  expect("fwd shape", efla_fwd_chunked(P, P, P, P, S, P, S, nullptr, 0, 2, 0, 100, 64, 64, 64, X, BF, nullptr),
         EFLA_ERR_BAD_SHAPE, 0);
  expect("fwd dk!=dv", efla_fwd_chunked(P, P, P, P, S, P, S, nullptr, 0, 2, 3, 100, 64, 32, 64, X, BF, nullptr),
         EFLA_ERR_BAD_SHAPE, 0);
  expect("fwd huge", efla_fwd_chunked(P, P, P, P, S, P, S, nullptr, 0, 1 << 16, 1 << 16, 100, 64, 64, 64, X, BF,
                                      nullptr), EFLA_ERR_BAD_SHAPE, 0);
  expect("fwd chunk", efla_fwd_chunked(P, P, P, P, S, P, S, nullptr, 0, 2, 3, 100, 64, 64, 48, X, BF, nullptr),
         EFLA_ERR_UNSUPPORTED, 0);
  expect("fwd coef", efla_fwd_chunked(P, P, P, P, S, P, S, nullptr, 0, 2, 3, 100, 64, 64, 64, (efla_coef)9, BF,
                                      nullptr), EFLA_ERR_UNSUPPORTED, 0);
  expect("fwd dtype", efla_fwd_chunked(P, P, P, P, S, P, S, nullptr, 0, 2, 3, 100, 64, 64, 64, X, (efla_dtype)5,
                                       nullptr), EFLA_ERR_UNSUPPORTED, 0);
  expect("fwd misaligned", efla_fwd_chunked(P, M, P, P, S, P, S, nullptr, 0, 2, 3, 100, 64, 64, 64, X, BF,
                                            nullptr), EFLA_ERR_MISALIGNED, 0);
  expect("fwd beta f32 misaligned", efla_fwd_chunked(P, P, P, M, S, P, S, nullptr, 0, 2, 3, 100, 64, 64, 64, X,
                                                     F32, nullptr), EFLA_ERR_MISALIGNED, 0);
  fwd_ws = 1024;
  expect("fwd workspace missing", efla_fwd_chunked(P, P, P, P, S, P, S, nullptr, 0, 2, 3, 100, 64, 64, 64, X,
                                                   BF, nullptr), EFLA_ERR_WORKSPACE, 0);
  expect("fwd workspace short", efla_fwd_chunked(P, P, P, P, S, P, S, P, 1023, 2, 3, 100, 64, 64, 64, X, BF,
                                                 nullptr), EFLA_ERR_WORKSPACE, 0);
  expect("fwd workspace ok", efla_fwd_chunked(P, P, P, P, S, P, S, P, 1024, 2, 3, 100, 64, 64, 64, X, BF,
                                              nullptr), EFLA_OK, 1);
  fwd_ws = 0;
  if (efla_fwd_chunked_workspace_bytes(2, 3, 100, 64, 64, 48, BF) != 0) ++fails;

  expect("step ok", efla_fwd_recurrent_step(P, P, P, P, S, P, 2, 3, 128, 128, X, BF, nullptr), EFLA_OK, 1);
  expect("step null", efla_fwd_recurrent_step(P, P, P, P, nullptr, P, 2, 3, 128, 128, X, BF, nullptr),
         EFLA_ERR_NULL_POINTER, 0);
  expect("step d", efla_fwd_recurrent_step(P, P, P, P, S, P, 2, 3, 96, 96, X, BF, nullptr), EFLA_ERR_UNSUPPORTED,
         0);
  expect("step misaligned", efla_fwd_recurrent_step(P, P, P, P, (float*)M, P, 2, 3, 128, 128, X, BF, nullptr),
         EFLA_ERR_MISALIGNED, 0);

  const float* G = (const float*)mem;
  expect("gated ok", efla_fwd_chunked_gated(P, P, P, P, G, S, P, S, 2, 3, 100, 128, 128, 64, X, F32, nullptr),
         EFLA_OK, 1);
  expect("gated null gate", efla_fwd_chunked_gated(P, P, P, P, nullptr, S, P, S, 2, 3, 100, 64, 64, 64, X, BF,
                                                   nullptr), EFLA_ERR_NULL_POINTER, 0);
  expect("gated gate misaligned", efla_fwd_chunked_gated(P, P, P, P, (const float*)M, S, P, S, 2, 3, 100, 64, 64,
                                                         64, X, BF, nullptr), EFLA_ERR_MISALIGNED, 0);
  expect("gated chunk", efla_fwd_chunked_gated(P, P, P, P, G, S, P, S, 2, 3, 100, 64, 64, 8, X, BF, nullptr),
         EFLA_ERR_UNSUPPORTED, 0);
  expect("gated step ok", efla_fwd_recurrent_step_gated(P, P, P, P, G, S, P, 2, 3, 64, 64, X, BF, nullptr), EFLA_OK,
         1);
  expect("gated step null", efla_fwd_recurrent_step_gated(P, P, P, P, nullptr, S, P, 2, 3, 64, 64, X, BF,
                                                          nullptr), EFLA_ERR_NULL_POINTER, 0);
  expect("bwd ok", efla_bwd_chunked(P, P, P, P, S, P, S, P, P, P, P, S, P, 64, 1, 2, 70, 32, 32, 32, X, BF,
                                    nullptr), EFLA_OK, 1);
  expect("bwd workspace", efla_bwd_chunked(P, P, P, P, S, P, S, P, P, P, P, S, P, 63, 1, 2, 70, 32, 32, 32, X,
                                           BF, nullptr), EFLA_ERR_WORKSPACE, 0);
  expect("bwd null", efla_bwd_chunked(P, P, P, P, S, P, S, nullptr, P, P, P, S, P, 64, 1, 2, 70, 32, 32, 32, X,
                                      BF, nullptr), EFLA_ERR_NULL_POINTER, 0);
  expect("saved ok", efla_bwd_chunked_saved(P, P, P, P, P, S, P, P, P, P, S, P, 64, 1, 2, 70, 32, 32, 32, X, BF,
                                            nullptr), EFLA_OK, 1);
  expect("train ok", efla_fwd_chunked_train(P, P, P, P, S, P, S, P, 64, 1, 2, 70, 32, 32, 32, X, BF, nullptr),
         EFLA_OK, 1);
  expect("train misaligned", efla_fwd_chunked_train(P, P, P, P, S, M, S, P, 64, 1, 2, 70, 32, 32, 32, X, BF,
                                                    nullptr), EFLA_ERR_MISALIGNED, 0);
  for (int s = -1; s <= 7; ++s)
    if (efla_status_string((efla_status)s) == nullptr) ++fails;
  printf("ABI sanitizer driver: %d failed checks\n", fails);
  return fails ? 1 : 0;
}
