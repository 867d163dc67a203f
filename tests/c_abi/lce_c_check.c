/*
 * lce_c_check.c - the library called through its C ABI alone: plain C, device
 * buffers from hipMalloc, the null stream, no Python and no torch.
 *
 * Test infrastructure.  Built by the package's build step with gcc against
 * include/lce.h and liblce.so; run by tests/test_c_abi_gpu.py on a GPU.
 *
 * Checks, bf16 inputs, 300 tokens, H = 64, V = 1000, strips of 256, mean
 * reduction, every tenth row ignored:
 *  1. W = 0.  Every logit is 0, so lse = ln V for every row, the loss is
 *     ln V, d_hidden = 0 exactly and d_weight row v is
 *     sum over valid rows i of (1/V - [t_i = v]) h_i / n_valid: the
 *     closed form of softmax minus one-hot at uniform probabilities.
 *  2. Random W.  The strip-level calls (lce_forward_begin / _fold / _end,
 *     lce_backward_begin / _fold) with the strips in reverse order give the
 *     same loss, lse, d_hidden and d_weight as lce_forward / lce_backward up
 *     to the order of fp32 sums (which can also flip the bf16 rounding of a
 *     few elements of G).
 * Exit status 0 when every check holds, 1 when one fails, 2 on an API or
 * runtime error.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "lce.h"

#define CHECK_HIP(x)                                                         \
  do {                                                                       \
    hipError_t e_ = (x);                                                     \
    if (e_ != hipSuccess) {                                                  \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));         \
      exit(2);                                                               \
    }                                                                        \
  } while (0)
#define CHECK_LCE(x)                                                         \
  do {                                                                       \
    lce_status_t s_ = (x);                                                   \
    if (s_ != LCE_OK) {                                                      \
      fprintf(stderr, "%s failed: %s\n", #x, lce_status_string(s_));         \
      exit(2);                                                               \
    }                                                                        \
  } while (0)

enum { N = 300, H = 64, V = 1000, VS = 256 };

static int failures = 0;
static void expect(int ok, const char* what, double value, double bound) {
  printf("%-44s %.3e (bound %.1e) %s\n", what, value, bound, ok ? "ok" : "FAILED");
  if (!ok) ++failures;
}

/* float -> bf16 bits, round to nearest even; bf16 bits -> float */
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* xorshift64 uniform numbers in [0, 1) */
static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double uniform(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return (double)(rng_state >> 11) / 9007199254740992.0;
}

struct Device {
  void *h, *w, *ws;
  int32_t* t;
  float *loss, *lse, *row_loss, *go, *dh, *dw;
  size_t ws_bytes;
};

static void run_whole(const lce_problem_t* p, struct Device* d) {
  CHECK_LCE(lce_forward(p, d->h, d->w, d->t, d->loss, d->lse, d->row_loss, d->ws, d->ws_bytes, 0));
  CHECK_LCE(lce_backward(p, d->h, d->w, d->t, d->lse, d->go, d->dh, d->dw, d->ws, d->ws_bytes, 0));
}

static void run_strips_reversed(const lce_problem_t* p, struct Device* d) {
  const int64_t n_strips = (V + VS - 1) / VS;
  CHECK_LCE(lce_forward_begin(p, d->ws, d->ws_bytes, 0));
  for (int64_t k = n_strips - 1; k >= 0; --k) {
    const int64_t v0 = k * VS, len = V - v0 < VS ? V - v0 : VS;
    CHECK_LCE(lce_forward_fold(p, d->h, (const uint16_t*)d->w + v0 * H, v0, len, d->t, d->ws,
                               d->ws_bytes, 0));
  }
  CHECK_LCE(lce_forward_end(p, d->t, d->loss, d->lse, d->row_loss, d->ws, d->ws_bytes, 0));
  CHECK_LCE(lce_backward_begin(p, d->t, d->go, d->ws, d->ws_bytes, 0));
  for (int64_t k = n_strips - 1; k >= 0; --k) {
    const int64_t v0 = k * VS, len = V - v0 < VS ? V - v0 : VS;
    const int acc = k == n_strips - 1 ? LCE_ACC_NONE : LCE_ACC_DHIDDEN;
    CHECK_LCE(lce_backward_fold(p, d->h, (const uint16_t*)d->w + v0 * H, v0, len, d->t, d->lse,
                                d->dh, acc, d->dw + v0 * H, d->ws, d->ws_bytes, 0));
  }
}

static void fetch(const struct Device* d, float* loss, float* lse, float* row_loss, float* dh,
                  float* dw) {
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(loss, d->loss, sizeof(float), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(lse, d->lse, N * sizeof(float), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(row_loss, d->row_loss, N * sizeof(float), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(dh, d->dh, (size_t)N * H * sizeof(float), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(dw, d->dw, (size_t)V * H * sizeof(float), hipMemcpyDeviceToHost));
}

int main(void) {
  const lce_problem_t p = {N, H, V, VS, LCE_BF16, LCE_MEAN, -100, 0};
  struct Device d;
  d.ws_bytes = lce_workspace_bytes(&p);
  if (d.ws_bytes == 0) {
    fprintf(stderr, "lce_workspace_bytes rejected the problem\n");
    return 2;
  }

  static uint16_t h[N * H], w[V * H];
  static int32_t t[N];
  static float hf[N * H];
  int n_valid = 0;
  for (int i = 0; i < N * H; ++i) {
    h[i] = to_bf16((float)(2.0 * uniform() - 1.0));
    hf[i] = from_bf16(h[i]);
  }
  for (int i = 0; i < N; ++i) {
    t[i] = i % 10 == 3 ? -100 : (int32_t)(uniform() * V);
    n_valid += t[i] != -100;
  }
  memset(w, 0, sizeof(w));

  CHECK_HIP(hipMalloc(&d.h, sizeof(h)));
  CHECK_HIP(hipMalloc(&d.w, sizeof(w)));
  CHECK_HIP(hipMalloc((void**)&d.t, sizeof(t)));
  CHECK_HIP(hipMalloc((void**)&d.loss, sizeof(float)));
  CHECK_HIP(hipMalloc((void**)&d.lse, N * sizeof(float)));
  CHECK_HIP(hipMalloc((void**)&d.row_loss, N * sizeof(float)));
  CHECK_HIP(hipMalloc((void**)&d.go, sizeof(float)));
  CHECK_HIP(hipMalloc((void**)&d.dh, (size_t)N * H * sizeof(float)));
  CHECK_HIP(hipMalloc((void**)&d.dw, (size_t)V * H * sizeof(float)));
  CHECK_HIP(hipMalloc(&d.ws, d.ws_bytes));
  const float one = 1.0f;
  CHECK_HIP(hipMemcpy(d.h, h, sizeof(h), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d.w, w, sizeof(w), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d.t, t, sizeof(t), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d.go, &one, sizeof(float), hipMemcpyHostToDevice));

  static float loss, lse[N], row_loss[N], dh[N * H], dw[V * H];
  static float loss2, lse2[N], row_loss2[N], dh2[N * H], dw2[V * H];

  /* 1. W = 0: closed forms */
  run_whole(&p, &d);
  fetch(&d, &loss, lse, row_loss, dh, dw);
  const double ln_v = log((double)V);
  double e_lse = 0.0, e_row = 0.0, max_dh = 0.0;
  for (int i = 0; i < N; ++i) {
    e_lse = fmax(e_lse, fabs(lse[i] - ln_v));
    e_row = fmax(e_row, fabs(row_loss[i] - (t[i] == -100 ? 0.0 : ln_v)));
  }
  for (int i = 0; i < N * H; ++i) max_dh = fmax(max_dh, fabs(dh[i]));
  double num = 0.0, den = 0.0;
  for (int v = 0; v < V; ++v)
    for (int k = 0; k < H; ++k) {
      double ref = 0.0;
      for (int i = 0; i < N; ++i)
        if (t[i] != -100) ref += (1.0 / V - (t[i] == v ? 1.0 : 0.0)) * hf[i * H + k] / n_valid;
      const double diff = dw[v * H + k] - ref;
      num += diff * diff;
      den += ref * ref;
    }
  expect(fabs(loss - ln_v) <= 2e-6 * ln_v, "W=0: |loss - ln V| / ln V", fabs(loss - ln_v) / ln_v, 2e-6);
  expect(e_lse <= 2e-5 * (1.0 + ln_v), "W=0: max |lse - ln V|", e_lse, 2e-5 * (1.0 + ln_v));
  expect(e_row <= 2e-5 * (1.0 + ln_v), "W=0: max |row loss - closed form|", e_row, 2e-5 * (1.0 + ln_v));
  expect(max_dh == 0.0, "W=0: max |d_hidden|", max_dh, 0.0);
  expect(sqrt(num / den) <= 1e-2, "W=0: d_weight rel. Frobenius error", sqrt(num / den), 1e-2);

  /* 2. random W: reversed strip-level calls against the whole passes */
  for (int i = 0; i < V * H; ++i) w[i] = to_bf16((float)(0.2 * uniform() - 0.1));
  CHECK_HIP(hipMemcpy(d.w, w, sizeof(w), hipMemcpyHostToDevice));
  run_whole(&p, &d);
  fetch(&d, &loss, lse, row_loss, dh, dw);
  run_strips_reversed(&p, &d);
  fetch(&d, &loss2, lse2, row_loss2, dh2, dw2);
  double d_lse = 0.0, d_dh = 0.0, n_dh = 0.0, d_dw = 0.0, n_dw = 0.0;
  for (int i = 0; i < N; ++i) d_lse = fmax(d_lse, fabs(lse2[i] - lse[i]));
  for (int i = 0; i < N * H; ++i) {
    d_dh += (double)(dh2[i] - dh[i]) * (dh2[i] - dh[i]);
    n_dh += (double)dh[i] * dh[i];
  }
  for (int i = 0; i < V * H; ++i) {
    d_dw += (double)(dw2[i] - dw[i]) * (dw2[i] - dw[i]);
    n_dw += (double)dw[i] * dw[i];
  }
  expect(fabs(loss2 - loss) <= 1e-6 * fabs(loss), "reversed strips: |d loss| / loss",
         fabs(loss2 - loss) / fabs(loss), 1e-6);
  expect(d_lse <= 1e-5, "reversed strips: max |d lse|", d_lse, 1e-5);
  expect(sqrt(d_dh / n_dh) <= 1e-4, "reversed strips: d_hidden rel. Frobenius diff",
         sqrt(d_dh / n_dh), 1e-4);
  expect(sqrt(d_dw / n_dw) <= 1e-4, "reversed strips: d_weight rel. Frobenius diff",
         sqrt(d_dw / n_dw), 1e-4);

  hipFree(d.h);
  hipFree(d.w);
  hipFree(d.t);
  hipFree(d.loss);
  hipFree(d.lse);
  hipFree(d.row_loss);
  hipFree(d.go);
  hipFree(d.dh);
  hipFree(d.dw);
  hipFree(d.ws);
  printf("c-abi check: %s (loss %.6f)\n", failures ? "FAILED" : "ok", loss);
  return failures ? 1 : 0;
}
