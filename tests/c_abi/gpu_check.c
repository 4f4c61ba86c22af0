/*
 * A C caller of libhsv.so on the GPU: device buffers from the HIP runtime
 * API, then hsv_verify_attn twice -- once with the parent array, once with
 * the ancestor bitmask that hsv_tree_ancestor_mask builds from it -- and a
 * comparison of both outputs with the reference values in the input file.
 *
 * Input file (little-endian), as the test writes it:
 *   int32 header[9]: B, N, Hq, Hkv, D, kv_capacity, in_dtype (0 fp32, 1 bf16),
 *                    max_ctx, magic 0x48535643
 *   q [B, N, Hq, D], k [B, Hkv, cap, D], v (in_dtype: 4 or 2 bytes each),
 *   ctx_lens int32 [B], parent int32 [B, N],
 *   o_ref float64 [B, N, Hq, D], lse_ref float64 [B, N, Hq].
 * Prints the largest errors of each call; exits 0 when both are within
 * max |dO| <= 1e-2 and max |dLSE| / max(|lse_ref|, 1) <= 1e-3 with the same
 * empty rows (lse = -inf), else 1 (2 on a usage or I/O error, 3 on a HIP or
 * library error).
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "hsv.h"

#define HIP_OK(call)                                                   \
  do {                                                                 \
    hipError_t e_ = (call);                                            \
    if (e_ != hipSuccess) {                                            \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));       \
      exit(3);                                                         \
    }                                                                  \
  } while (0)

#define HSV_OK(call)                                                   \
  do {                                                                 \
    hsv_status s_ = (call);                                            \
    if (s_ != HSV_OK) {                                                \
      fprintf(stderr, "%s: %s\n", #call, hsv_status_string(s_));       \
      exit(3);                                                         \
    }                                                                  \
  } while (0)

static void *read_block(FILE *f, size_t bytes) {
  void *p = malloc(bytes ? bytes : 1);
  if (!p || fread(p, 1, bytes, f) != bytes) {
    fprintf(stderr, "input file too short\n");
    exit(2);
  }
  return p;
}

static void *to_device(const void *host, size_t bytes) {
  void *d = NULL;
  HIP_OK(hipMalloc(&d, bytes ? bytes : 1));
  if (bytes) HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

/* Largest errors of one call's output against the reference; 1 if within
 * the bar, 0 if not. */
static int compare(const char *what, const float *o, const float *lse, const double *o_ref,
                   const double *lse_ref, size_t n_rows, int D) {
  double o_err = 0.0, l_err = 0.0;
  int pattern_ok = 1, finite = 1;
  for (size_t r = 0; r < n_rows; ++r) {
    const int ref_empty = isinf(lse_ref[r]) && lse_ref[r] < 0;
    const int got_empty = isinf(lse[r]) && lse[r] < 0;
    if (ref_empty != got_empty) pattern_ok = 0;
    if (!ref_empty) {
      const double den = fabs(lse_ref[r]) > 1.0 ? fabs(lse_ref[r]) : 1.0;
      const double e = fabs((double)lse[r] - lse_ref[r]) / den;
      if (e > l_err) l_err = e;
    }
    for (int d = 0; d < D; ++d) {
      const float x = o[r * (size_t)D + d];
      if (!isfinite(x)) finite = 0;
      const double e = fabs((double)x - o_ref[r * (size_t)D + d]);
      if (e > o_err) o_err = e;
    }
  }
  printf("%s: max|dO|=%.3e max rel dLSE=%.3e%s%s\n", what, o_err, l_err,
         pattern_ok ? "" : " (empty rows differ)", finite ? "" : " (non-finite output)");
  return pattern_ok && finite && o_err <= 1e-2 && l_err <= 1e-3;
}

int main(int argc, char **argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s INPUT\n", argv[0]);
    return 2;
  }
  FILE *f = fopen(argv[1], "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", argv[1]);
    return 2;
  }
  int32_t h[9];
  if (fread(h, sizeof h, 1, f) != 1 || h[8] != 0x48535643) {
    fprintf(stderr, "bad header\n");
    return 2;
  }
  const int B = h[0], N = h[1], Hq = h[2], Hkv = h[3], D = h[4], cap = h[5], in_dt = h[6];
  const int max_ctx = h[7];
  const size_t el = in_dt == HSV_BF16 ? 2 : 4;
  const size_t n_q = (size_t)B * N * Hq * D, n_kv = (size_t)B * Hkv * cap * D;
  const size_t n_rows = (size_t)B * N * Hq;
  void *q = read_block(f, n_q * el), *k = read_block(f, n_kv * el), *v = read_block(f, n_kv * el);
  int32_t *ctx = (int32_t *)read_block(f, (size_t)B * sizeof(int32_t));
  int32_t *parent = (int32_t *)read_block(f, (size_t)B * N * sizeof(int32_t));
  double *o_ref = (double *)read_block(f, n_q * sizeof(double));
  double *lse_ref = (double *)read_block(f, n_rows * sizeof(double));
  fclose(f);

  hsv_verify_desc d;
  memset(&d, 0, sizeof d);
  d.batch = B;
  d.n_draft = N;
  d.n_q_heads = Hq;
  d.n_kv_heads = Hkv;
  d.head_dim = D;
  d.kv_capacity = cap;
  d.max_ctx = max_ctx;
  d.in_dtype = in_dt;
  d.out_dtype = HSV_F32;
  size_t ws_bytes = 0;
  HSV_OK(hsv_verify_workspace_bytes(&d, &ws_bytes));

  void *dq = to_device(q, n_q * el), *dk = to_device(k, n_kv * el), *dv = to_device(v, n_kv * el);
  int32_t *dctx = (int32_t *)to_device(ctx, (size_t)B * sizeof(int32_t));
  int32_t *dpar = (int32_t *)to_device(parent, (size_t)B * N * sizeof(int32_t));
  const int words = (N + 63) / 64;
  uint64_t *danc = NULL;
  float *dlse = NULL;
  void *dout = NULL, *dws = NULL;
  HIP_OK(hipMalloc((void **)&danc, (size_t)B * N * words * sizeof(uint64_t)));
  HIP_OK(hipMalloc(&dout, n_q * sizeof(float)));
  HIP_OK(hipMalloc((void **)&dlse, n_rows * sizeof(float)));
  HIP_OK(hipMalloc(&dws, ws_bytes ? ws_bytes : 1));
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));

  float *o = (float *)malloc(n_q * sizeof(float));
  float *lse = (float *)malloc(n_rows * sizeof(float));
  if (!o || !lse) return 2;
  int ok = 1;

  /* 1. the parent array */
  HSV_OK(hsv_verify_attn(&d, dq, dk, dv, dctx, dpar, NULL, dout, dlse, dws, ws_bytes, stream));
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(o, dout, n_q * sizeof(float), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(lse, dlse, n_rows * sizeof(float), hipMemcpyDeviceToHost));
  ok &= compare("parent array", o, lse, o_ref, lse_ref, n_rows, D);

  /* 2. the ancestor bitmask built on the device from the same parents */
  HSV_OK(hsv_tree_ancestor_mask(dpar, danc, B, N, stream));
  HSV_OK(hsv_verify_attn(&d, dq, dk, dv, dctx, NULL, danc, dout, dlse, dws, ws_bytes, stream));
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(o, dout, n_q * sizeof(float), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(lse, dlse, n_rows * sizeof(float), hipMemcpyDeviceToHost));
  ok &= compare("ancestor bitmask", o, lse, o_ref, lse_ref, n_rows, D);

  HIP_OK(hipStreamDestroy(stream));
  HIP_OK(hipFree(dq));
  HIP_OK(hipFree(dk));
  HIP_OK(hipFree(dv));
  HIP_OK(hipFree(dctx));
  HIP_OK(hipFree(dpar));
  HIP_OK(hipFree(danc));
  HIP_OK(hipFree(dout));
  HIP_OK(hipFree(dlse));
  HIP_OK(hipFree(dws));
  free(q);
  free(k);
  free(v);
  free(ctx);
  free(parent);
  free(o_ref);
  free(lse_ref);
  free(o);
  free(lse);
  printf(ok ? "all checks passed\n" : "checks failed\n");
  return ok ? 0 : 1;
}
