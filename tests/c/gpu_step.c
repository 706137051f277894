/* One outer step on the GPU through the C ABI alone: the HIP runtime for device
 * memory, libdlc for the work, no Python.
 *
 *  - Tensors 0-2 (ragged sizes) are moved by every learner by an exact dyadic
 *    constant c_i: each pseudo-gradient is constant, its quantization is the
 *    zero-variance case (every code 0, the codebook holds the mean c_i), and the
 *    merge g = sum_i w_hat_i c_i is exact.  theta and momentum must equal the
 *    Nesterov step (v <- beta v + g; theta <- theta - lr (g + beta v)) evaluated
 *    here in double in the same order, bit for bit.
 *  - Tensor 3 holds pseudo-random (near-Gaussian) pseudo-gradients: every bucket that received an element
 *    has its codebook entry inside the bucket [lo + c wd, lo + (c + 1) wd].
 *  - dlc_quantize_static writes the same codes, codebook and range as
 *    dlc_quantize with a caller's workspace.
 * Prints "ok <checks>" and exits 0, or names the first failure and exits 1. */
#include <hip/hip_runtime_api.h>

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dlc.h"

#define K 3
#define T 4

static int checks = 0;

static void fail(const char* what) {
  printf("FAIL %s\n", what);
  exit(1);
}

static void hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    printf("FAIL %s: %s\n", what, hipGetErrorString(e));
    exit(1);
  }
}

static void dlc_ok(int32_t rc, const char* what) {
  if (rc != DLC_OK) {
    printf("FAIL %s: %d %s\n", what, (int)rc, dlc_last_error());
    exit(1);
  }
}

static void expect(int cond, const char* what) {
  ++checks;
  if (!cond) fail(what);
}

/* xorshift64*: a uniform double in (0, 1) */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform(void) {
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return ((double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) + 0.5) / 9007199254740992.0;
}

/* sum of twelve uniforms minus 6: mean 0, variance 1, tails to +-6 */
static double near_normal(void) {
  double s = -6.0;
  for (int j = 0; j < 12; ++j) s += uniform();
  return s;
}

int main(void) {
  const int64_t numel[T] = {5000, 64, 4097, 100003};
  dlc_tensor tensors[T];
  int64_t pos = 0;
  for (int t = 0; t < T; ++t) {
    tensors[t].offset = pos;
    tensors[t].loffset = pos;
    tensors[t].numel = numel[t];
    pos += (numel[t] + DLC_ALIGN_ELEMS - 1) / DLC_ALIGN_ELEMS * DLC_ALIGN_ELEMS;
  }
  const int64_t stride = pos;
  const double c[K] = {0x1p-10, -0x1p-11, 0x3p-12};
  const double weights[K] = {1.0, 2.0, 1.0}; /* w_hat = 1/4, 1/2, 1/4 */
  const double lr = 0.7, beta = 0.9;

  float* theta = (float*)malloc(sizeof(float) * stride);
  float* mom = (float*)malloc(sizeof(float) * stride);
  float* learners = (float*)malloc(sizeof(float) * K * stride);
  if (!theta || !mom || !learners) fail("host allocation");
  memset(theta, 0, sizeof(float) * stride);
  memset(mom, 0, sizeof(float) * stride);
  memset(learners, 0, sizeof(float) * K * stride);
  for (int t = 0; t < T; ++t) {
    for (int64_t e = 0; e < numel[t]; ++e) {
      const int64_t o = tensors[t].offset + e;
      if (t < 3) {
        theta[o] = 0.5f;
        mom[o] = 0x1p-8f;
        for (int i = 0; i < K; ++i) learners[i * stride + o] = (float)(0.5 - c[i]);
      } else {
        theta[o] = (float)(0.04 * (uniform() - 0.5));
        for (int i = 0; i < K; ++i) learners[i * stride + o] = theta[o] - (float)(1e-3 * near_normal());
      }
    }
  }

  float *d_theta, *d_mom, *d_learners, *d_cb, *d_rng, *d_cb2, *d_rng2;
  uint8_t *d_codes, *d_codes2;
  void* d_ws;
  size_t ws_bytes = 0;
  dlc_ok(dlc_workspace_bytes(K, tensors, T, &ws_bytes), "dlc_workspace_bytes");
  hip_ok(hipMalloc((void**)&d_theta, sizeof(float) * stride), "hipMalloc theta");
  hip_ok(hipMalloc((void**)&d_mom, sizeof(float) * stride), "hipMalloc momentum");
  hip_ok(hipMalloc((void**)&d_learners, sizeof(float) * K * stride), "hipMalloc learners");
  hip_ok(hipMalloc((void**)&d_codes, (size_t)K * stride), "hipMalloc codes");
  hip_ok(hipMalloc((void**)&d_codes2, (size_t)K * stride), "hipMalloc codes");
  hip_ok(hipMalloc((void**)&d_cb, sizeof(float) * K * T * DLC_N_BUCKETS), "hipMalloc codebook");
  hip_ok(hipMalloc((void**)&d_cb2, sizeof(float) * K * T * DLC_N_BUCKETS), "hipMalloc codebook");
  hip_ok(hipMalloc((void**)&d_rng, sizeof(float) * K * T * DLC_RANGE_FIELDS), "hipMalloc range");
  hip_ok(hipMalloc((void**)&d_rng2, sizeof(float) * K * T * DLC_RANGE_FIELDS), "hipMalloc range");
  hip_ok(hipMalloc(&d_ws, ws_bytes), "hipMalloc workspace");
  hip_ok(hipMemcpy(d_theta, theta, sizeof(float) * stride, hipMemcpyHostToDevice), "copy theta");
  hip_ok(hipMemcpy(d_mom, mom, sizeof(float) * stride, hipMemcpyHostToDevice), "copy momentum");
  hip_ok(hipMemcpy(d_learners, learners, sizeof(float) * K * stride, hipMemcpyHostToDevice), "copy learners");
  /* the alignment gaps between tensors are never written: clear both code buffers */
  hip_ok(hipMemset(d_codes, 0, (size_t)K * stride), "clear codes");
  hip_ok(hipMemset(d_codes2, 0, (size_t)K * stride), "clear codes");

  dlc_ok(dlc_quantize(d_theta, d_learners, stride, K, NULL, tensors, T, d_codes, d_cb, d_rng, 0, d_ws, ws_bytes,
                      NULL),
         "dlc_quantize");
  dlc_ok(dlc_quantize_static(d_theta, d_learners, stride, K, NULL, tensors, T, d_codes2, d_cb2, d_rng2, 0, NULL),
         "dlc_quantize_static");
  dlc_ok(dlc_merge_outer_step(d_theta, d_mom, d_codes, stride, K, d_cb, weights, tensors, T, lr, beta, 0, NULL),
         "dlc_merge_outer_step");
  hip_ok(hipDeviceSynchronize(), "synchronize");

  uint8_t* codes = (uint8_t*)malloc((size_t)K * stride);
  uint8_t* codes2 = (uint8_t*)malloc((size_t)K * stride);
  float* cb = (float*)malloc(sizeof(float) * K * T * DLC_N_BUCKETS);
  float* cb2 = (float*)malloc(sizeof(float) * K * T * DLC_N_BUCKETS);
  float* rng = (float*)malloc(sizeof(float) * K * T * DLC_RANGE_FIELDS);
  float* rng2 = (float*)malloc(sizeof(float) * K * T * DLC_RANGE_FIELDS);
  float* theta_out = (float*)malloc(sizeof(float) * stride);
  float* mom_out = (float*)malloc(sizeof(float) * stride);
  if (!codes || !codes2 || !cb || !cb2 || !rng || !rng2 || !theta_out || !mom_out) fail("host allocation");
  hip_ok(hipMemcpy(codes, d_codes, (size_t)K * stride, hipMemcpyDeviceToHost), "copy codes");
  hip_ok(hipMemcpy(codes2, d_codes2, (size_t)K * stride, hipMemcpyDeviceToHost), "copy codes");
  hip_ok(hipMemcpy(cb, d_cb, sizeof(float) * K * T * DLC_N_BUCKETS, hipMemcpyDeviceToHost), "copy codebook");
  hip_ok(hipMemcpy(cb2, d_cb2, sizeof(float) * K * T * DLC_N_BUCKETS, hipMemcpyDeviceToHost), "copy codebook");
  hip_ok(hipMemcpy(rng, d_rng, sizeof(float) * K * T * DLC_RANGE_FIELDS, hipMemcpyDeviceToHost), "copy range");
  hip_ok(hipMemcpy(rng2, d_rng2, sizeof(float) * K * T * DLC_RANGE_FIELDS, hipMemcpyDeviceToHost), "copy range");
  hip_ok(hipMemcpy(theta_out, d_theta, sizeof(float) * stride, hipMemcpyDeviceToHost), "copy theta");
  hip_ok(hipMemcpy(mom_out, d_mom, sizeof(float) * stride, hipMemcpyDeviceToHost), "copy momentum");

  /* the static scratch call equals the workspace call */
  expect(memcmp(codes, codes2, (size_t)K * stride) == 0, "static codes differ");
  expect(memcmp(cb, cb2, sizeof(float) * K * T * DLC_N_BUCKETS) == 0, "static codebook differs");
  expect(memcmp(rng, rng2, sizeof(float) * K * T * DLC_RANGE_FIELDS) == 0, "static range differs");

  /* constant tensors: exact quantization and the Nesterov step in double */
  double g = 0.0;
  for (int i = 0; i < K; ++i) g += weights[i] / 4.0 * c[i];
  for (int t = 0; t < 3; ++t) {
    for (int i = 0; i < K; ++i) {
      const float* r = rng + ((size_t)i * T + t) * DLC_RANGE_FIELDS;
      expect(r[3] == (float)c[i], "mean of a constant tensor");
      expect(cb[((size_t)i * T + t) * DLC_N_BUCKETS] == (float)c[i], "codebook entry 0 of a constant tensor");
      for (int64_t e = 0; e < numel[t]; ++e) {
        if (codes[i * stride + tensors[t].loffset + e] != 0) fail("code of a constant tensor");
      }
      ++checks;
    }
    const double bv = beta * (double)0x1p-8f;
    const double vn = bv + g;
    const double step = g + beta * vn;
    const float want_v = (float)vn, want_t = (float)(0.5 - lr * step);
    for (int64_t e = 0; e < numel[t]; ++e) {
      const int64_t o = tensors[t].offset + e;
      if (mom_out[o] != want_v) fail("momentum of a constant tensor");
      if (theta_out[o] != want_t) fail("theta of a constant tensor");
    }
    checks += 2;
  }

  /* the pseudo-random tensor: every used codebook entry lies inside its bucket */
  for (int i = 0; i < K; ++i) {
    const float* r = rng + ((size_t)i * T + 3) * DLC_RANGE_FIELDS;
    expect(isfinite(r[0]) && isfinite(r[1]) && r[0] < r[1] && r[2] > 0.0f, "range of the random tensor");
    int64_t count[DLC_N_BUCKETS];
    memset(count, 0, sizeof(count));
    for (int64_t e = 0; e < numel[3]; ++e) ++count[codes[i * stride + tensors[3].loffset + e]];
    int used = 0;
    for (int b = 0; b < DLC_N_BUCKETS; ++b) {
      if (count[b] == 0) continue;
      ++used;
      const double lo = (double)r[0] + b * (double)r[2], hi = lo + (double)r[2];
      const double v = (double)cb[((size_t)i * T + 3) * DLC_N_BUCKETS + b];
      const double slack = 1e-6 * (double)r[2];
      if (!(v >= lo - slack && v <= hi + slack)) fail("codebook entry outside its bucket");
      ++checks;
    }
    expect(used > 100, "the random tensor uses most buckets");
  }

  printf("ok %d\n", checks);
  return 0;
}
