/* A plain C caller of the library's C ABI (include/conv1d_gn.h), with the HIP
 * runtime's C API for device memory and a stream.  For each case it builds the
 * descriptors, checks them and asks for the route, sizes and allocates the
 * workspace, runs conv1d_gn_forward on its own stream, and compares the
 * output and the exported statistics with the fp64 oracle's C functions
 * (test infrastructure, linked in only here).  It also checks that an invalid
 * call is refused with a status before anything runs.  Built and run by
 * tests/test_c_abi.py; exit status 0 when every case is within 1e-4. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "conv1d_gn.h"

/* the oracle's entry points (oracle/oracle.c) */
int64_t oracle_out_len(int64_t T, int64_t K, int64_t stride, int64_t dilation, int64_t pad_left,
                       int64_t pad_right);
void oracle_conv1d(int64_t N, int64_t C_in, int64_t C_out, int64_t T, int64_t K, int64_t stride,
                   int64_t dilation, int64_t pad_left, int64_t pad_right, const double* x,
                   const double* w, const double* bias, double* y);
void oracle_group_norm(int64_t N, int64_t C, int64_t L, int64_t G, double eps, const double* y,
                       const double* gamma, const double* beta, double* z, double* mean_out,
                       double* rstd_out);
void oracle_layer_norm_channels(int64_t N, int64_t C, int64_t L, double eps, const double* y,
                                const double* gamma, const double* beta, double* z,
                                double* mean_out, double* rstd_out);

#define HIP_OK(call)                                                        \
  do {                                                                      \
    hipError_t e_ = (call);                                                 \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));            \
      exit(2);                                                              \
    }                                                                       \
  } while (0)

/* uniform values in [-1, 1) from a 64-bit linear congruential generator */
static float draw(uint64_t* s) {
  *s = *s * 6364136223846793005ull + 1442695040888963407ull;
  return (float)((double)(*s >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}

static float* device_copy(const float* h, size_t n) {
  void* d = NULL;
  HIP_OK(hipMalloc(&d, n * sizeof(float)));
  HIP_OK(hipMemcpy(d, h, n * sizeof(float), hipMemcpyHostToDevice));
  return (float*)d;
}

/* one conv1d + normalisation call against the oracle; returns 0 on success */
static int run_case(const char* name, c1g_conv_desc d, c1g_norm_desc nd, uint64_t seed) {
  const int64_t T_out = c1g_out_len(&d);
  if (T_out != oracle_out_len(d.T, d.K, d.stride, d.dilation, d.pad_left, d.pad_right)) {
    printf("%s: T_out %lld disagrees with the oracle\n", name, (long long)T_out);
    return 1;
  }
  const size_t nx = (size_t)(d.N * d.C_in * d.T), nw = (size_t)(d.C_out * d.C_in * d.K);
  const size_t no = (size_t)(d.N * d.C_out * T_out);
  const size_t ns = (size_t)(nd.norm == C1G_NORM_GROUP ? d.N * nd.G : d.N * T_out);
  float *x = malloc(nx * sizeof(float)), *w = malloc(nw * sizeof(float));
  float *b = malloc(d.C_out * sizeof(float)), *ga = malloc(d.C_out * sizeof(float));
  float *be = malloc(d.C_out * sizeof(float)), *out = malloc(no * sizeof(float));
  float *mean = malloc(ns * sizeof(float)), *rstd = malloc(ns * sizeof(float));
  for (size_t i = 0; i < nx; ++i) x[i] = draw(&seed);
  for (size_t i = 0; i < nw; ++i) w[i] = draw(&seed) * 0.2f;
  for (int64_t c = 0; c < d.C_out; ++c) {
    b[c] = draw(&seed) * 0.1f;
    ga[c] = 1.0f + 0.5f * draw(&seed);
    be[c] = draw(&seed) * 0.1f;
  }

  int st = c1g_check(&d, &nd, (size_t)-1);
  if (st != C1G_OK) {
    printf("%s: c1g_check: %s\n", name, c1g_status_string(st));
    return 1;
  }
  const size_t ws_bytes = c1g_conv1d_gn_workspace_size(&d, &nd);
  void* ws = NULL;
  if (ws_bytes) HIP_OK(hipMalloc(&ws, ws_bytes));  /* 256-byte aligned */
  float *dx = device_copy(x, nx), *dw = device_copy(w, nw), *db = device_copy(b, d.C_out);
  float *dga = device_copy(ga, d.C_out), *dbe = device_copy(be, d.C_out);
  void *dout = NULL, *dmean = NULL, *drstd = NULL;
  HIP_OK(hipMalloc(&dout, no * sizeof(float)));
  HIP_OK(hipMalloc(&dmean, ns * sizeof(float)));
  HIP_OK(hipMalloc(&drstd, ns * sizeof(float)));
  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  st = conv1d_gn_forward(&d, &nd, dx, dw, db, dga, dbe, NULL, dout, (float*)dmean,
                         (float*)drstd, ws, ws_bytes, (void*)s);
  if (st != C1G_OK) {
    printf("%s: conv1d_gn_forward: %s\n", name, c1g_status_string(st));
    return 1;
  }
  HIP_OK(hipStreamSynchronize(s));
  HIP_OK(hipMemcpy(out, dout, no * sizeof(float), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(mean, dmean, ns * sizeof(float), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(rstd, drstd, ns * sizeof(float), hipMemcpyDeviceToHost));

  /* the oracle on the same values, widened to fp64 */
  double *xd = malloc(nx * sizeof(double)), *wd = malloc(nw * sizeof(double));
  double *bd = malloc(d.C_out * sizeof(double)), *gd = malloc(d.C_out * sizeof(double));
  double *ed = malloc(d.C_out * sizeof(double)), *y = malloc(no * sizeof(double));
  double *z = malloc(no * sizeof(double)), *md = malloc(ns * sizeof(double));
  double *rd = malloc(ns * sizeof(double));
  for (size_t i = 0; i < nx; ++i) xd[i] = x[i];
  for (size_t i = 0; i < nw; ++i) wd[i] = w[i];
  for (int64_t c = 0; c < d.C_out; ++c) {
    bd[c] = b[c];
    gd[c] = ga[c];
    ed[c] = be[c];
  }
  oracle_conv1d(d.N, d.C_in, d.C_out, d.T, d.K, d.stride, d.dilation, d.pad_left, d.pad_right,
                xd, wd, bd, y);
  if (nd.norm == C1G_NORM_GROUP)
    oracle_group_norm(d.N, d.C_out, T_out, nd.G, nd.eps, y, gd, ed, z, md, rd);
  else
    oracle_layer_norm_channels(d.N, d.C_out, T_out, nd.eps, y, gd, ed, z, md, rd);
  double err = 0.0, merr = 0.0, rerr = 0.0;
  for (size_t i = 0; i < no; ++i) {
    const double e = fabs((double)out[i] - z[i]);
    err = (e > err || e != e) ? e : err;
  }
  for (size_t i = 0; i < ns; ++i) {
    const double em = fabs((double)mean[i] - md[i]), er = fabs((double)rstd[i] / rd[i] - 1.0);
    merr = (em > merr || em != em) ? em : merr;
    rerr = (er > rerr || er != er) ? er : rerr;
  }
  const int ok = err <= 1e-4 && merr <= 1e-4 && rerr <= 1e-4;
  printf("%-24s route %-18s ws %8zu B  max|out - oracle| %.3g  mean %.3g  rstd (rel) %.3g  %s\n",
         name, c1g_route(&d, &nd), ws_bytes, err, merr, rerr, ok ? "ok" : "FAIL");

  HIP_OK(hipStreamDestroy(s));
  HIP_OK(hipFree(dx));
  HIP_OK(hipFree(dw));
  HIP_OK(hipFree(db));
  HIP_OK(hipFree(dga));
  HIP_OK(hipFree(dbe));
  HIP_OK(hipFree(dout));
  HIP_OK(hipFree(dmean));
  HIP_OK(hipFree(drstd));
  if (ws) HIP_OK(hipFree(ws));
  free(x); free(w); free(b); free(ga); free(be); free(out); free(mean); free(rstd);
  free(xd); free(wd); free(bd); free(gd); free(ed); free(y); free(z); free(md); free(rd);
  return ok ? 0 : 1;
}

int main(void) {
  int fails = 0;
  /* fused single pass: fp32, GroupNorm, symmetric padding */
  c1g_conv_desc d1 = {3, 24, 64, 300, 3, 1, 1, 1, 1, C1G_F32, C1G_F32, C1G_LAYOUT_NCL};
  c1g_norm_desc n1 = {C1G_NORM_GROUP, 8, 1e-5f, C1G_EPI_NONE, 0};
  fails += run_case("fused_gn_fp32", d1, n1, 1);
  /* split: fp32, LayerNorm over channels, causal dilated conv past 1024 positions */
  c1g_conv_desc d2 = {2, 16, 40, 1500, 4, 1, 2, 6, 0, C1G_F32, C1G_F32, C1G_LAYOUT_NCL};
  c1g_norm_desc n2 = {C1G_NORM_LAYER_CHANNELS, 0, 1e-5f, C1G_EPI_NONE, 0};
  fails += run_case("split_ln_fp32_causal", d2, n2, 2);

  /* an invalid call is refused before anything runs: C_out not divisible by G */
  c1g_norm_desc bad = {C1G_NORM_GROUP, 7, 1e-5f, C1G_EPI_NONE, 0};
  const int st = conv1d_gn_forward(&d1, &bad, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                   NULL, NULL, 0, NULL);
  printf("C_out %% G != 0: %s\n", c1g_status_string(st));
  if (st != C1G_ERR_INVALID_ARG) ++fails;

  printf(fails ? "FAIL\n" : "OK\n");
  return fails ? 1 : 0;
}
