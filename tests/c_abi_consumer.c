/* A plain C99 program that uses libvjp through include/libvjp.h and the HIP
 * runtime's C API only (no C++, no Python, no torch): it allocates device
 * buffers, calls one entry point of each op family, and checks the results
 * against closed forms that need no reference implementation:
 *   weighted sum of x[i][j] = (i+1)(j+1) with w = 1: y_i = (i+1) d(d+1)/2,
 *     grad_x = dy (w = 1), grad_w_j = (j+1) n(n+1)/2 for dy = 1 (all exact);
 *   softmax: every row of y sums to 1; a row-constant dy gives dx = 0;
 *   softmax cross-entropy of all-zero logits: loss = row_lse = ln C,
 *     dlogits = scale (1/C - [j = target]);
 *   scaled SiLU at x = 0: y = 0, dx = w dy / 2, dw = 0 (also through the
 *     no-allocation entry point);
 *   row gather of table rows holding their own index: y[m] = idx[m]; the
 *     backward of dy = 1 gives each row its selection count; invalid
 *     indices are counted;
 *   a device copy; an invalid argument's status and message.
 * Prints one line per check and exits non-zero if any fails. */
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "libvjp.h"

static int failures = 0;

#define HIP_OK(call)                                                               \
  do {                                                                             \
    hipError_t e_ = (call);                                                        \
    if (e_ != hipSuccess) {                                                        \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));                   \
      exit(2);                                                                     \
    }                                                                              \
  } while (0)

#define VJP_OK_CALL(call)                                                          \
  do {                                                                             \
    int s_ = (call);                                                               \
    if (s_ != VJP_OK) {                                                            \
      fprintf(stderr, "%s: %s (%s)\n", #call, vjp_status_string(s_), vjp_last_error()); \
      exit(3);                                                                     \
    }                                                                              \
  } while (0)

static void report(const char* name, int ok, double worst) {
  printf("%-44s %s (worst %.3g)\n", name, ok ? "ok" : "FAILED", worst);
  if (!ok) ++failures;
}

static void* dev_alloc(size_t bytes) {
  void* p = NULL;
  HIP_OK(hipMalloc(&p, bytes > 0 ? bytes : 1));
  return p;
}

static void to_dev(void* d, const void* h, size_t bytes) {
  HIP_OK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
}

static void to_host(void* h, const void* d, size_t bytes) {
  HIP_OK(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
}

static void check_weighted_sum(void) {
  const int64_t n = 100, d = 64;
  float* x = malloc(sizeof(float) * n * d);
  float* w = malloc(sizeof(float) * d);
  float* dy = malloc(sizeof(float) * n);
  float* y = malloc(sizeof(float) * n);
  float* dx = malloc(sizeof(float) * n * d);
  float* dw = malloc(sizeof(float) * d);
  for (int64_t i = 0; i < n; ++i)
    for (int64_t j = 0; j < d; ++j) x[i * d + j] = (float)((i + 1) * (j + 1));
  for (int64_t j = 0; j < d; ++j) w[j] = 1.0f;
  for (int64_t i = 0; i < n; ++i) dy[i] = 1.0f;
  float *xd = dev_alloc(sizeof(float) * n * d), *wd = dev_alloc(sizeof(float) * d);
  float *dyd = dev_alloc(sizeof(float) * n), *yd = dev_alloc(sizeof(float) * n);
  float *dxd = dev_alloc(sizeof(float) * n * d), *dwd = dev_alloc(sizeof(float) * d);
  const size_t wsb = vjp_weighted_sum_bwd_workspace_size(n, d, 32);
  void* ws = dev_alloc(wsb);
  to_dev(xd, x, sizeof(float) * n * d);
  to_dev(wd, w, sizeof(float) * d);
  to_dev(dyd, dy, sizeof(float) * n);
  VJP_OK_CALL(vjp_weighted_sum_fwd(xd, d, wd, yd, n, d, VJP_F32, VJP_F32, NULL));
  VJP_OK_CALL(vjp_weighted_sum_bwd(dyd, xd, d, wd, dxd, d, dwd, 0, n, d, 32, VJP_F32, VJP_F32,
                                   ws, wsb, NULL));
  HIP_OK(hipDeviceSynchronize());
  to_host(y, yd, sizeof(float) * n);
  to_host(dx, dxd, sizeof(float) * n * d);
  to_host(dw, dwd, sizeof(float) * d);
  double worst = 0.0;
  int ok = 1;
  for (int64_t i = 0; i < n; ++i) {
    const double want = (double)(i + 1) * d * (d + 1) / 2;
    worst = fmax(worst, fabs(y[i] - want));
    ok &= y[i] == (float)want;
  }
  report("weighted_sum y (exact)", ok, worst);
  ok = 1;
  for (int64_t k = 0; k < n * d; ++k) ok &= dx[k] == 1.0f;
  report("weighted_sum grad_x (exact)", ok, 0.0);
  ok = 1;
  worst = 0.0;
  for (int64_t j = 0; j < d; ++j) {
    const double want = (double)(j + 1) * n * (n + 1) / 2;
    worst = fmax(worst, fabs(dw[j] - want));
    ok &= dw[j] == (float)want;
  }
  report("weighted_sum grad_w (exact)", ok, worst);
  HIP_OK(hipFree(xd)); HIP_OK(hipFree(wd)); HIP_OK(hipFree(dyd)); HIP_OK(hipFree(yd));
  HIP_OK(hipFree(dxd)); HIP_OK(hipFree(dwd)); HIP_OK(hipFree(ws));
  free(x); free(w); free(dy); free(y); free(dx); free(dw);
}

static void check_softmax(void) {
  const int64_t rows = 64, cols = 1000;
  float* x = malloc(sizeof(float) * rows * cols);
  float* dy = malloc(sizeof(float) * rows * cols);
  float* y = malloc(sizeof(float) * rows * cols);
  unsigned s = 12345u;
  for (int64_t k = 0; k < rows * cols; ++k) {
    s = s * 1664525u + 1013904223u;
    x[k] = (float)((s >> 8) % 2001) / 250.0f - 4.0f;   /* in [-4, 4] */
  }
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) dy[r * cols + c] = (float)(r % 7) - 3.0f;
  float *xd = dev_alloc(sizeof(float) * rows * cols), *yd = dev_alloc(sizeof(float) * rows * cols);
  float *dyd = dev_alloc(sizeof(float) * rows * cols), *dxd = dev_alloc(sizeof(float) * rows * cols);
  to_dev(xd, x, sizeof(float) * rows * cols);
  to_dev(dyd, dy, sizeof(float) * rows * cols);
  VJP_OK_CALL(vjp_softmax_fwd(xd, cols, yd, cols, rows, cols, VJP_F32, NULL));
  VJP_OK_CALL(vjp_softmax_bwd(dyd, cols, yd, cols, dxd, cols, rows, cols, VJP_F32, NULL));
  HIP_OK(hipDeviceSynchronize());
  to_host(y, yd, sizeof(float) * rows * cols);
  double worst = 0.0;
  for (int64_t r = 0; r < rows; ++r) {
    double sum = 0.0;
    for (int64_t c = 0; c < cols; ++c) sum += y[r * cols + c];
    worst = fmax(worst, fabs(sum - 1.0));
  }
  report("softmax rows of y sum to 1", worst <= 1e-5, worst);
  to_host(y, dxd, sizeof(float) * rows * cols);   /* dx */
  worst = 0.0;
  for (int64_t k = 0; k < rows * cols; ++k) worst = fmax(worst, fabs(y[k]));
  report("softmax dx = 0 for a row-constant dy", worst <= 1e-6, worst);
  HIP_OK(hipFree(xd)); HIP_OK(hipFree(yd)); HIP_OK(hipFree(dyd)); HIP_OK(hipFree(dxd));
  free(x); free(dy); free(y);
}

static void check_xent(void) {
  const int64_t rows = 32, C = 1000;
  const float scale = 1.0f / (float)rows;
  float* z = calloc((size_t)(rows * C), sizeof(float));
  float* dz = malloc(sizeof(float) * rows * C);
  float* lse = malloc(sizeof(float) * rows);
  int32_t* t = malloc(sizeof(int32_t) * rows);
  for (int64_t r = 0; r < rows; ++r) t[r] = (int32_t)((r * 37) % C);
  float *zd = dev_alloc(sizeof(float) * rows * C), *dzd = dev_alloc(sizeof(float) * rows * C);
  float *lossd = dev_alloc(sizeof(float)), *maxd = dev_alloc(sizeof(float) * rows);
  float *lsed = dev_alloc(sizeof(float) * rows);
  int32_t *td = dev_alloc(sizeof(int32_t) * rows), *ninvd = dev_alloc(sizeof(int32_t));
  const size_t wsb = vjp_softmax_xent_workspace_size(rows);
  void* ws = dev_alloc(wsb);
  to_dev(zd, z, sizeof(float) * rows * C);
  to_dev(td, t, sizeof(int32_t) * rows);
  VJP_OK_CALL(vjp_softmax_xent_fwd_bwd(zd, C, td, rows, C, VJP_F32, scale, lossd, maxd, lsed, dzd,
                                       C, ninvd, ws, wsb, NULL));
  HIP_OK(hipDeviceSynchronize());
  float loss = 0.0f;
  int32_t ninv = -1;
  to_host(&loss, lossd, sizeof(float));
  to_host(&ninv, ninvd, sizeof(int32_t));
  to_host(lse, lsed, sizeof(float) * rows);
  to_host(dz, dzd, sizeof(float) * rows * C);
  const double lnC = log((double)C);
  double worst = fabs(loss - lnC);
  for (int64_t r = 0; r < rows; ++r) worst = fmax(worst, fabs(lse[r] - lnC));
  report("xent loss = row_lse = ln C for zero logits", worst <= 1e-5 * lnC && ninv == 0, worst);
  worst = 0.0;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < C; ++c) {
      const double want = scale * (1.0 / C - (c == t[r] ? 1.0 : 0.0));
      worst = fmax(worst, fabs(dz[r * C + c] - want) / fabs(want));
    }
  report("xent dlogits = scale (1/C - onehot)", worst <= 1e-5, worst);
  HIP_OK(hipFree(zd)); HIP_OK(hipFree(dzd)); HIP_OK(hipFree(lossd)); HIP_OK(hipFree(maxd));
  HIP_OK(hipFree(lsed)); HIP_OK(hipFree(td)); HIP_OK(hipFree(ninvd)); HIP_OK(hipFree(ws));
  free(z); free(dz); free(lse); free(t);
}

static void check_silu(void) {
  const int64_t n = 10007;
  const float wv = 0.75f;
  float* x = calloc((size_t)n, sizeof(float));
  float* dy = malloc(sizeof(float) * n);
  float* out = malloc(sizeof(float) * n);
  for (int64_t k = 0; k < n; ++k) dy[k] = (float)(k % 11) - 5.0f;
  float *xd = dev_alloc(sizeof(float) * n), *dyd = dev_alloc(sizeof(float) * n);
  float *yd = dev_alloc(sizeof(float) * n), *dxd = dev_alloc(sizeof(float) * n);
  float *wd = dev_alloc(sizeof(float)), *dwd = dev_alloc(sizeof(float));
  const size_t wsb = vjp_scaled_silu_bwd_workspace_size(n);
  void* ws = dev_alloc(wsb);
  to_dev(xd, x, sizeof(float) * n);
  to_dev(dyd, dy, sizeof(float) * n);
  to_dev(wd, &wv, sizeof(float));
  VJP_OK_CALL(vjp_scaled_silu_fwd(xd, wd, yd, n, VJP_F32, NULL));
  HIP_OK(hipDeviceSynchronize());
  to_host(out, yd, sizeof(float) * n);
  int ok = 1;
  for (int64_t k = 0; k < n; ++k) ok &= out[k] == 0.0f;
  report("scaled_silu y = 0 at x = 0", ok, 0.0);
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 0)
      VJP_OK_CALL(vjp_scaled_silu_bwd(dyd, xd, wd, dxd, dwd, 0, n, VJP_F32, ws, wsb, NULL));
    else
      VJP_OK_CALL(vjp_scaled_silu_bwd_noalloc(dyd, xd, wd, dxd, dwd, 0, n, VJP_F32, NULL));
    HIP_OK(hipDeviceSynchronize());
    float dw = -1.0f;
    to_host(out, dxd, sizeof(float) * n);
    to_host(&dw, dwd, sizeof(float));
    ok = dw == 0.0f;
    for (int64_t k = 0; k < n; ++k) ok &= out[k] == 0.5f * wv * dy[k];
    report(pass == 0 ? "scaled_silu dx = w dy / 2, dw = 0 at x = 0"
                     : "the same through the no-allocation entry point",
           ok, 0.0);
  }
  HIP_OK(hipFree(xd)); HIP_OK(hipFree(dyd)); HIP_OK(hipFree(yd)); HIP_OK(hipFree(dxd));
  HIP_OK(hipFree(wd)); HIP_OK(hipFree(dwd)); HIP_OK(hipFree(ws));
  free(x); free(dy); free(out);
}

static void check_gather(void) {
  const int64_t V = 50, D = 64, M = 1000;
  float* table = malloc(sizeof(float) * V * D);
  float* y = malloc(sizeof(float) * M * D);
  float* dy = malloc(sizeof(float) * M * D);
  float* dt = malloc(sizeof(float) * V * D);
  int32_t* idx = malloc(sizeof(int32_t) * M);
  int64_t count[50] = {0};
  int32_t invalid = 0;
  for (int64_t v = 0; v < V; ++v)
    for (int64_t c = 0; c < D; ++c) table[v * D + c] = (float)v;
  for (int64_t m = 0; m < M; ++m) {
    idx[m] = (m % 97 == 0) ? -1 : (int32_t)((m * m + 3) % V);   /* repeats and a few invalid */
    if (idx[m] < 0) ++invalid; else ++count[idx[m]];
  }
  for (int64_t k = 0; k < M * D; ++k) dy[k] = 1.0f;
  float *td = dev_alloc(sizeof(float) * V * D), *yd = dev_alloc(sizeof(float) * M * D);
  float *dyd = dev_alloc(sizeof(float) * M * D), *dtd = dev_alloc(sizeof(float) * V * D);
  int32_t *idxd = dev_alloc(sizeof(int32_t) * M), *ninvd = dev_alloc(sizeof(int32_t));
  const size_t wsb = vjp_gather_rows_bwd_workspace_size(M, V, D);
  void* ws = dev_alloc(wsb);
  to_dev(td, table, sizeof(float) * V * D);
  to_dev(idxd, idx, sizeof(int32_t) * M);
  to_dev(dyd, dy, sizeof(float) * M * D);
  VJP_OK_CALL(vjp_gather_rows_fwd(td, D, V, D, idxd, M, yd, D, VJP_F32, NULL));
  VJP_OK_CALL(vjp_gather_rows_bwd(dyd, D, idxd, M, V, D, dtd, D, 0, ninvd, VJP_F32, ws, wsb, NULL));
  HIP_OK(hipDeviceSynchronize());
  to_host(y, yd, sizeof(float) * M * D);
  to_host(dt, dtd, sizeof(float) * V * D);
  int32_t ninv = -1;
  to_host(&ninv, ninvd, sizeof(int32_t));
  int ok = 1;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t c = 0; c < D; ++c) ok &= y[m * D + c] == (idx[m] < 0 ? 0.0f : (float)idx[m]);
  report("gather y[m] = table[idx[m]] (0 when invalid)", ok, 0.0);
  ok = ninv == invalid;
  for (int64_t v = 0; v < V; ++v)
    for (int64_t c = 0; c < D; ++c) ok &= dt[v * D + c] == (float)count[v];
  report("scatter-add rows = selection counts", ok, 0.0);
  HIP_OK(hipFree(td)); HIP_OK(hipFree(yd)); HIP_OK(hipFree(dyd)); HIP_OK(hipFree(dtd));
  HIP_OK(hipFree(idxd)); HIP_OK(hipFree(ninvd)); HIP_OK(hipFree(ws));
  free(table); free(y); free(dy); free(dt); free(idx);
}

static void check_copy_and_errors(void) {
  const int64_t bytes = (1 << 20) + 13;
  unsigned char* a = malloc((size_t)bytes);
  unsigned char* b = malloc((size_t)bytes);
  for (int64_t k = 0; k < bytes; ++k) a[k] = (unsigned char)(k * 131 + 7);
  void *ad = dev_alloc((size_t)bytes), *bd = dev_alloc((size_t)bytes);
  to_dev(ad, a, (size_t)bytes);
  VJP_OK_CALL(vjp_copy(ad, bd, bytes, NULL));
  HIP_OK(hipDeviceSynchronize());
  to_host(b, bd, (size_t)bytes);
  report("copy of 1 MiB + 13 bytes", memcmp(a, b, (size_t)bytes) == 0, 0.0);
  const int s = vjp_softmax_fwd(ad, 16, bd, 16, -1, 16, VJP_F32, NULL);
  const char* msg = vjp_last_error();
  report("invalid size: VJP_EINVAL with a message",
         s == VJP_EINVAL && msg != NULL && msg[0] != '\0' && vjp_status_string(s) != NULL, 0.0);
  HIP_OK(hipFree(ad)); HIP_OK(hipFree(bd));
  free(a); free(b);
}

int main(void) {
  printf("libvjp version %d\n", vjp_version());
  check_weighted_sum();
  check_softmax();
  check_xent();
  check_silu();
  check_gather();
  check_copy_and_errors();
  printf("%s\n", failures == 0 ? "all checks passed" : "some checks FAILED");
  return failures == 0 ? 0 : 1;
}
