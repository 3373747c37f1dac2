// Host-only driver for the argument checks and the workspace planner; built
// with AddressSanitizer and UndefinedBehaviorSanitizer by the CPU tests.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <initializer_list>
#include <limits>

#include "flce.h"

static int failures = 0;
#define EXPECT(cond)                                              \
  do {                                                            \
    if (!(cond)) { std::printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #cond); ++failures; } \
  } while (0)

static int call(int64_t N, int64_t H, int64_t V, int dtype, int red, int64_t T, float s,
                float mb, size_t wsb, uintptr_t ws = uintptr_t(1) << 40) {
  const uintptr_t b = uintptr_t(1) << 32;
  return flce_check_args((void*)b, (void*)(b * 2), (int64_t*)(b * 3), N, H, V, -100, s, red, T,
                         (float*)(b * 4), (int64_t*)(b * 5), (void*)(b * 6), (void*)(b * 7),
                         nullptr, dtype, mb, 0, (void*)ws, wsb, nullptr, nullptr);
}

static int fcall(int64_t N, int64_t H, int64_t V, int dtype, int red, int64_t T, float s,
                 size_t wsb) {
  const uintptr_t b = uintptr_t(1) << 32;
  return flce_forward_check_args((void*)b, (void*)(b * 2), (int64_t*)(b * 3), N, H, V, -100, s,
                                 red, T, (float*)(b * 4), (int64_t*)(b * 5), nullptr, dtype, 1.f,
                                 (void*)(uintptr_t(1) << 40), wsb, nullptr, nullptr);
}

int main() {
  const size_t big = size_t(1) << 40;
  EXPECT(call(8192, 4096, 131072, FLCE_BF16, FLCE_MEAN, 0, 0.f, 1.f, big) == FLCE_OK);
  EXPECT(call(8192, 4096, 131072, FLCE_BF16, FLCE_MEAN, 5, 0.f, 1.f, big) == FLCE_ERR_ARG);
  EXPECT(call(1, 12, 5, FLCE_BF16, FLCE_SUM, 0, 0.f, 1.f, big) == FLCE_OK);   // padded to 16
  EXPECT(call(1, 12, 5, FLCE_F32, FLCE_SUM, 0, 0.f, 1.f, big) == FLCE_OK);
  EXPECT(call(1, 8, 5, FLCE_BF16, FLCE_SUM, 0, -0.5f, 1.f, big) == FLCE_ERR_ARG);
  EXPECT(call(1, 8, 5, FLCE_BF16, FLCE_SUM, 0, std::numeric_limits<float>::quiet_NaN(), 1.f,
              big) == FLCE_ERR_ARG);
  EXPECT(call(1, 8, 5, FLCE_BF16, FLCE_SUM, 0, 0.f, INFINITY, big) == FLCE_ERR_ARG);
  EXPECT(call(1, 8, 5, FLCE_BF16, FLCE_SUM, 0, 0.f, 1.f, 10) == FLCE_ERR_WORKSPACE);
  EXPECT(call(1, 8, 5, FLCE_BF16, FLCE_SUM, 0, 0.f, 1.f, big, (uintptr_t(1) << 40) + 16) ==
         FLCE_ERR_WORKSPACE);
  // a gradient output sharing memory with the workspace (dW holds intermediate
  // values during the call) or with another argument is refused
  const uintptr_t b = uintptr_t(1) << 32;
  EXPECT(call(1, 8, 5, FLCE_BF16, FLCE_SUM, 0, 0.f, 1.f, big, b * 7 - 256) == FLCE_ERR_ARG);
  EXPECT(call(1, 8, 5, FLCE_BF16, FLCE_SUM, 0, 0.f, 1.f, 256, b * 6 + 8) == FLCE_ERR_ARG);
  EXPECT(call(1, 8, 5, FLCE_BF16, FLCE_SUM, 0, 0.f, 1.f, big, b * 8) == FLCE_OK);
  EXPECT(flce_check_args((void*)b, (void*)(b * 2), (int64_t*)(b * 7), 1, 8, 5, -100, 0.f,
                         FLCE_SUM, 0, (float*)(b * 4), (int64_t*)(b * 5), (void*)(b * 6),
                         (void*)(b * 7), nullptr, FLCE_BF16, 1.f, 0, (void*)(b * 8), big, nullptr,
                         nullptr) == FLCE_ERR_ARG);                 // labels inside dW
  EXPECT(flce_check_args((void*)b, (void*)(b * 2), (int64_t*)(b * 3), 1, 8, 5, -100, 0.f,
                         FLCE_SUM, 0, (float*)(b * 4), (int64_t*)(b * 5), (void*)(b * 6),
                         (void*)(b * 7), nullptr, FLCE_BF16, 1.f, 0, (void*)(b * 8), big,
                         (int32_t*)(b * 6 + 8), nullptr) == FLCE_ERR_ARG);   // status inside dH
  // extreme sizes are refused, never overflow
  EXPECT(call(int64_t(1) << 40, 8, 5, FLCE_BF16, FLCE_SUM, 0, 0.f, 1.f, big) == FLCE_ERR_ARG);
  EXPECT(call(8, int64_t(1) << 40, 5, FLCE_BF16, FLCE_SUM, 0, 0.f, 1.f, big) == FLCE_ERR_ARG);
  EXPECT(flce_workspace_size(INT64_MAX, INT64_MAX, INT64_MAX, FLCE_BF16) == 0);
  for (int64_t n : {0, 1, 7, 255, 256, 257, 4096, 16384})
    for (int64_t v : {1, 2, 255, 256, 257, 32000, 131072, 256000}) {
      const size_t w = flce_workspace_size(n, 64, v, FLCE_BF16);
      EXPECT(w > 0 && w % 256 == 0);
      const int64_t c = flce_vocab_chunk(n, 64, v, FLCE_BF16);
      EXPECT(c >= 256 && c % 256 == 0);
      // a hidden size that is not a multiple of 8: padded copies carved too
      const size_t wo = flce_workspace_size(n, 61, v, FLCE_BF16);
      EXPECT(wo % 256 == 0 && (n == 0 ? wo == w : wo > w));
      EXPECT(flce_forward_workspace_size(n, 61, v, FLCE_BF16) % 256 == 0);
    }
  // forward-only entry: same rules, its own (smaller) workspace
  EXPECT(fcall(8192, 4096, 131072, FLCE_BF16, FLCE_MEAN, 0, 0.f, big) == FLCE_OK);
  EXPECT(fcall(8192, 4096, 131072, FLCE_BF16, FLCE_MEAN, 5, 0.f, big) == FLCE_ERR_ARG);
  EXPECT(fcall(int64_t(1) << 40, 8, 5, FLCE_BF16, FLCE_SUM, 0, 0.f, big) == FLCE_ERR_ARG);
  EXPECT(flce_forward_workspace_size(INT64_MAX, INT64_MAX, INT64_MAX, FLCE_BF16) == 0);
  for (int64_t n : {0, 1, 257, 16384})
    for (int64_t v : {1, 257, 256000}) {
      const size_t f = flce_forward_workspace_size(n, 64, v, FLCE_BF16);
      const size_t w = flce_workspace_size(n, 64, v, FLCE_BF16);
      EXPECT(f > 0 && f % 256 == 0 && (n > 0 ? f < w : f == w));
      EXPECT(fcall(n, 64, v, FLCE_BF16, FLCE_SUM, 0, 0.f, f) == FLCE_OK);
      EXPECT(fcall(n, 64, v, FLCE_BF16, FLCE_SUM, 0, 0.f, f - 1) == FLCE_ERR_WORKSPACE);
    }
  // float32 gradients for bf16 inputs
  {
    const uintptr_t b = uintptr_t(1) << 32;
    auto ex = [&](int dtype, int grad, size_t wsb) {
      return flce_check_args_ex((void*)b, (void*)(b * 2), (int64_t*)(b * 3), 4096, 4096, 131072,
                                -100, 0.f, FLCE_SUM, 0, (float*)(b * 4), (int64_t*)(b * 5),
                                (void*)(b * 6), (void*)(b * 8), nullptr, dtype, 1.f, 0,
                                (void*)(uintptr_t(1) << 40), wsb, nullptr, nullptr, grad);
    };
    EXPECT(ex(FLCE_BF16, FLCE_F32, big) == FLCE_OK);
    EXPECT(ex(FLCE_F32, FLCE_BF16, big) == FLCE_ERR_UNSUPPORTED);
    EXPECT(ex(FLCE_BF16, 9, big) == FLCE_ERR_ARG);
    const size_t w = flce_workspace_size_ex(4096, 4096, 131072, FLCE_BF16, FLCE_F32);
    EXPECT(w > 0 && ex(FLCE_BF16, FLCE_F32, w) == FLCE_OK && ex(FLCE_BF16, FLCE_F32, w - 1) == FLCE_ERR_WORKSPACE);
    EXPECT(flce_vocab_chunk_ex(4096, 4096, 131072, FLCE_BF16, FLCE_F32) * 2 ==
           flce_vocab_chunk(4096, 4096, 131072, FLCE_BF16));
  }
  // logits-returning forward: sizes at the limits are refused or accepted
  // without overflow in the overlap arithmetic
  {
    const uintptr_t b = uintptr_t(1) << 32;
    auto lc = [&](int64_t N, int64_t V, int64_t ld, int ldt, uintptr_t lg) {
      return flce_forward_logits_check_args(
          (void*)b, (void*)(b * 2), (int64_t*)(b * 3), N, 8, V, -100, 0.f, FLCE_SUM, 0,
          (float*)(b * 4), (int64_t*)(b * 5), nullptr, FLCE_F32, 1.f,
          (void*)(uintptr_t(1) << 40), big, nullptr, nullptr, (void*)lg, ld, ldt);
    };
    const uintptr_t far = uintptr_t(1) << 50;
    EXPECT(lc(1024, 1000, 1000, FLCE_F32, far) == FLCE_OK);
    EXPECT(lc(1024, 1000, 999, FLCE_F32, far) == FLCE_ERR_ARG);
    EXPECT(lc(int64_t(1) << 31, int64_t(1) << 31, int64_t(1) << 31, FLCE_F32, far) ==
           FLCE_ERR_ARG);
    EXPECT(lc((int64_t(1) << 29) + 2, 1 << 20, int64_t(1) << 31, FLCE_BF16, far) == FLCE_ERR_ARG);
    EXPECT(lc(int64_t(1) << 29, 8, int64_t(1) << 31, FLCE_BF16, far) == FLCE_OK);
    EXPECT(lc(4, 7, INT64_MAX, FLCE_F32, far) == FLCE_ERR_ARG);
    EXPECT(lc(4, 7, 7, FLCE_BF16, far + 1) == FLCE_ERR_UNSUPPORTED);
    EXPECT(lc(4, 7, 7, FLCE_F32, b * 3) == FLCE_ERR_ARG);   // on the labels
    EXPECT(lc(0, 7, 7, FLCE_F32, 0) == FLCE_OK);
  }
  for (int s = -1; s < 8; ++s) EXPECT(flce_status_string(s) != nullptr);
  if (failures == 0) std::printf("all checks passed\n");
  return failures ? 1 : 0;
}
