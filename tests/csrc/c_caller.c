/*
 * A plain C caller of the fused linear cross-entropy library: device memory
 * and copies through the HIP runtime, no PyTorch, no C++.
 *
 * With W = 0 every logit is 0, so the result has a closed form (token-level
 * cross-entropy with ignore_index and 'sum'/'mean', NeMo AutoModel linear_ce
 * page, "API"; num_tokens, twinkle PR 335, "PR information", item 1):
 *   lse_t = ln V for every token, the loss of a kept token ln V,
 *   loss = n_kept ln V ('sum') or ln V ('mean'),
 *   num_tokens = n_kept ('sum') or 0 ('mean'),
 *   G[t][v] = c (1/V - [v = y_t]) for a kept token (c = 1 for 'sum',
 *   1 / n_kept for 'mean'), 0 for an ignored one,
 *   dH = G W = 0 exactly, dW[v] = sum_t G[t][v] h[t].
 * The program checks each of them, for a hidden size that is a multiple of 8
 * and one that is not, and prints "c caller: all checks passed".
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "flce.h"

#define HIP_OK(x)                                                           \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x,             \
              hipGetErrorString(e_));                                       \
      exit(2);                                                              \
    }                                                                       \
  } while (0)

static int failures = 0;
#define CHECK(cond, ...)                                                    \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "FAILED %s: ", #cond);                                \
      fprintf(stderr, __VA_ARGS__);                                         \
      fprintf(stderr, "\n");                                                \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

static uint64_t rng_state;
static double uniform01(void) {    /* 64-bit LCG (Knuth's MMIX constants) */
  rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(rng_state >> 11) * (1.0 / 9007199254740992.0);
}

static uint16_t to_bf16(float f) {  /* round to nearest even; inputs finite */
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static void run_case(int64_t N, int64_t H, int64_t V, int reduction, uint64_t seed) {
  const int64_t ignore = -100;
  rng_state = seed;
  uint16_t* h = malloc((size_t)(N * H) * 2);
  int64_t* y = malloc((size_t)N * 8);
  int64_t kept = 0;
  for (int64_t i = 0; i < N * H; ++i) h[i] = to_bf16((float)(2.0 * uniform01() - 1.0));
  for (int64_t t = 0; t < N; ++t) {
    y[t] = (t % 7 == 3) ? ignore : (int64_t)(uniform01() * (double)V) % V;
    kept += y[t] != ignore;
  }

  void *dh, *dW_in, *dy, *ddH, *ddW, *dws, *dloss, *dnt, *dstatus, *dlse;
  const size_t ws_bytes = flce_workspace_size(N, H, V, FLCE_BF16);
  CHECK(ws_bytes > 0, "workspace size");
  HIP_OK(hipMalloc(&dh, (size_t)(N * H) * 2));
  HIP_OK(hipMalloc(&dW_in, (size_t)(V * H) * 2));
  HIP_OK(hipMalloc(&dy, (size_t)N * 8));
  HIP_OK(hipMalloc(&ddH, (size_t)(N * H) * 2));
  HIP_OK(hipMalloc(&ddW, (size_t)(V * H) * 2));
  HIP_OK(hipMalloc(&dws, ws_bytes));
  HIP_OK(hipMalloc(&dloss, 4));
  HIP_OK(hipMalloc(&dnt, 8));
  HIP_OK(hipMalloc(&dstatus, 4));
  HIP_OK(hipMalloc(&dlse, (size_t)N * 4));
  HIP_OK(hipMemcpy(dh, h, (size_t)(N * H) * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dy, y, (size_t)N * 8, hipMemcpyHostToDevice));
  HIP_OK(hipMemset(dW_in, 0, (size_t)(V * H) * 2));
  HIP_OK(hipMemset(ddH, 0xFF, (size_t)(N * H) * 2));   /* NaN: every row must be written */
  HIP_OK(hipMemset(ddW, 0xFF, (size_t)(V * H) * 2));
  HIP_OK(hipDeviceSynchronize());

  int rc = flce_check_args(dh, dW_in, dy, N, H, V, ignore, 0.f, reduction, 0, dloss, dnt, ddH,
                           ddW, NULL, FLCE_BF16, 1.f, 0, dws, ws_bytes, dstatus, dlse);
  CHECK(rc == FLCE_OK, "check_args returned %s", flce_status_string(rc));
  rc = flce_forward_backward(dh, dW_in, dy, N, H, V, ignore, 0.f, reduction, 0, dloss, dnt, ddH,
                             ddW, NULL, FLCE_BF16, 1.f, 0, dws, ws_bytes, dstatus, dlse);
  CHECK(rc == FLCE_OK, "forward_backward returned %s", flce_status_string(rc));
  HIP_OK(hipDeviceSynchronize());

  float loss;
  int64_t nt;
  int32_t status;
  float* lse = malloc((size_t)N * 4);
  uint16_t* dH = malloc((size_t)(N * H) * 2);
  uint16_t* dW = malloc((size_t)(V * H) * 2);
  HIP_OK(hipMemcpy(&loss, dloss, 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&nt, dnt, 8, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&status, dstatus, 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(lse, dlse, (size_t)N * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(dH, ddH, (size_t)(N * H) * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(dW, ddW, (size_t)(V * H) * 2, hipMemcpyDeviceToHost));

  const double lnV = log((double)V);
  const int mean = reduction == FLCE_MEAN;
  const double want_loss = mean ? lnV : (double)kept * lnV;
  CHECK(status == FLCE_OK, "status %d", (int)status);
  CHECK(nt == (mean ? 0 : kept), "num_tokens %lld, kept %lld", (long long)nt, (long long)kept);
  CHECK(fabs(loss - want_loss) <= 1e-5 * want_loss, "loss %.9g, want %.9g", loss, want_loss);
  for (int64_t t = 0; t < N; ++t)
    CHECK(fabs(lse[t] - lnV) <= 1e-5 * lnV, "lse[%lld] %.9g, want %.9g", (long long)t, lse[t],
          lnV);
  int64_t nonzero = 0;
  for (int64_t i = 0; i < N * H; ++i) nonzero += from_bf16(dH[i]) != 0.f;
  CHECK(nonzero == 0, "%lld elements of dH are not 0", (long long)nonzero);

  /* dW[v][k] = c (S[k] / V - sum over kept t with y_t = v of h[t][k]), S the
     sum of the kept rows */
  const double c = mean ? 1.0 / (double)kept : 1.0;
  double* S = calloc((size_t)H, sizeof(double));
  double* ref = calloc((size_t)(V * H), sizeof(double));
  for (int64_t t = 0; t < N; ++t) {
    if (y[t] == ignore) continue;
    for (int64_t k = 0; k < H; ++k) {
      const double x = from_bf16(h[t * H + k]);
      S[k] += x;
      ref[y[t] * H + k] -= x;
    }
  }
  double max_ref = 0.0, max_err = 0.0;
  for (int64_t v = 0; v < V; ++v)
    for (int64_t k = 0; k < H; ++k) {
      const double r = c * (S[k] / (double)V + ref[v * H + k]);
      const double g = from_bf16(dW[v * H + k]);
      max_ref = fmax(max_ref, fabs(r));
      max_err = isnan(g) ? INFINITY : fmax(max_err, fabs(g - r));
    }
  CHECK(max_err <= 2e-2 * max_ref, "dW max err %.3g, max ref %.3g", max_err, max_ref);
  printf("case N=%lld H=%lld V=%lld %s: loss %.7g (want %.7g), dW max err / max ref %.2e\n",
         (long long)N, (long long)H, (long long)V, mean ? "mean" : "sum", loss, want_loss,
         max_err / max_ref);

  free(S); free(ref); free(lse); free(dH); free(dW); free(h); free(y);
  HIP_OK(hipFree(dh)); HIP_OK(hipFree(dW_in)); HIP_OK(hipFree(dy)); HIP_OK(hipFree(ddH));
  HIP_OK(hipFree(ddW)); HIP_OK(hipFree(dws)); HIP_OK(hipFree(dloss)); HIP_OK(hipFree(dnt));
  HIP_OK(hipFree(dstatus)); HIP_OK(hipFree(dlse));
}

int main(void) {
  run_case(300, 64, 1000, FLCE_SUM, 11);
  run_case(257, 37, 515, FLCE_MEAN, 12);
  if (failures) {
    printf("c caller: %d checks failed\n", failures);
    return 1;
  }
  printf("c caller: all checks passed\n");
  return 0;
}
