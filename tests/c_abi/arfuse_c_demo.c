/*
 * Plain-C use of the arfuse C ABI, with no Python and no PyTorch in the
 * process: device buffers from hipMalloc, fused calls on a HIP stream, and
 * the results compared with the CPU oracle (linked from oracle/, which only
 * tests may do).
 *
 * Cases: N = 4, t = 3, d = 1040 with bf16 and FP4 outputs; N = 8, t = 2,
 * d = 8192 with bf16 and FP8 outputs; argument errors that must be rejected
 * before anything is enqueued. Exit status 0 when every check holds.
 *
 * Inputs are bf16 bit patterns drawn directly (random sign, exponent in a
 * narrow range, random mantissa) from a counter hash, so the generator does
 * no rounding of its own.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "arfuse.h"
#include "arfuse_oracle.h"

#define CHECK_HIP(x)                                                        \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "[c-demo] %s failed: %d\n", #x, (int)e_);             \
      exit(2);                                                              \
    }                                                                       \
  } while (0)

/* splitmix64 of a counter */
static uint64_t mix(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* bf16 bits: sign random, exponent 124..130 (|x| in [2^-3, 2^4)), 7 random
 * mantissa bits */
static uint16_t gen_bf16(uint64_t ctr) {
  const uint64_t r = mix(ctr);
  const uint16_t sign = (uint16_t)((r & 1u) << 15);
  const uint16_t exp = (uint16_t)(124u + (uint16_t)((r >> 1) % 7u));
  const uint16_t man = (uint16_t)((r >> 8) & 0x7Fu);
  return (uint16_t)(sign | (exp << 7) | man);
}

/* gamma in [0.5, 2): exponent 126 or 127, random mantissa */
static float gen_gamma(uint64_t ctr) {
  const uint64_t r = mix(ctr);
  const uint32_t bits = ((126u + (uint32_t)(r & 1u)) << 23) | (uint32_t)((r >> 9) & 0x7FFFFFu);
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

static int failures = 0;

static void expect(int ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "[c-demo] FAILED: %s\n", what);
    ++failures;
  }
}

/* One fused call on the device against the oracle. epi: ARFUSE_EPI_* mask of
 * the norm outputs besides residual_out (BF16 always, plus FP4 or FP8).
 * split_auto: let the library split the rows (workspace from hipMalloc and
 * filled with a garbage byte: it needs no clearing), make the call twice on
 * that workspace, and check the status word the split call must have. */
static void run_case(int n, int64_t t, int64_t d, int epi, uint64_t seed, hipStream_t stream,
                     int split_auto) {
  const int64_t e = t * d;
  const int fp4 = (epi & ARFUSE_EPI_FP4) != 0, fp8 = (epi & ARFUSE_EPI_FP8) != 0;
  const float eps = 1e-5f, inv_scale = 8.0f;
  uint16_t* h_parts = malloc((size_t)(n * e) * 2);
  uint16_t* h_res = malloc((size_t)e * 2);
  float* h_gamma = malloc((size_t)d * 4);
  for (int64_t i = 0; i < n * e; ++i) h_parts[i] = gen_bf16(seed + (uint64_t)i);
  for (int64_t i = 0; i < e; ++i) h_res[i] = gen_bf16(seed + 0x100000000ull + (uint64_t)i);
  for (int64_t j = 0; j < d; ++j) h_gamma[j] = gen_gamma(seed + 0x200000000ull + (uint64_t)j);

  void* d_parts[8];
  void *d_res, *d_gamma, *d_out, *d_rout, *d_codes = NULL, *d_scales = NULL, *d_fp8 = NULL;
  for (int i = 0; i < n; ++i) {
    CHECK_HIP(hipMalloc(&d_parts[i], (size_t)e * 2));
    CHECK_HIP(hipMemcpy(d_parts[i], h_parts + i * e, (size_t)e * 2, hipMemcpyHostToDevice));
  }
  CHECK_HIP(hipMalloc(&d_res, (size_t)e * 2));
  CHECK_HIP(hipMemcpy(d_res, h_res, (size_t)e * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMalloc(&d_gamma, (size_t)d * 4));
  CHECK_HIP(hipMemcpy(d_gamma, h_gamma, (size_t)d * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMalloc(&d_out, (size_t)e * 2));
  CHECK_HIP(hipMalloc(&d_rout, (size_t)e * 2));
  if (fp4) {
    CHECK_HIP(hipMalloc(&d_codes, (size_t)e / 2));
    CHECK_HIP(hipMalloc(&d_scales, (size_t)e / 16));
  }
  if (fp8) CHECK_HIP(hipMalloc(&d_fp8, (size_t)e));

  int rc;
  void* d_ws = NULL;
  arfuse_ll_status* d_status = NULL;
  if (split_auto) {
    arfuse_opts o;
    memset(&o, 0, sizeof o);
    o.split = ARFUSE_SPLIT_AUTO;
    arfuse_launch_info info;
    expect(arfuse_query_launch(n, t, d, epi, &o, &info) == ARFUSE_OK, "query of the automatic split");
    printf("[c-demo] automatic split for n=%d t=%lld d=%lld: %d workgroups per row, workspace %lld bytes\n",
           n, (long long)t, (long long)d, info.split, (long long)info.workspace_bytes);
    if (info.workspace_bytes > 0) {
      CHECK_HIP(hipMalloc(&d_ws, (size_t)info.workspace_bytes));
      CHECK_HIP(hipMemset(d_ws, 0xA5, (size_t)info.workspace_bytes));
    }
    CHECK_HIP(hipMalloc((void**)&d_status, sizeof(arfuse_ll_status)));
    CHECK_HIP(hipMemset(d_status, 0, sizeof(arfuse_ll_status)));
    o.workspace = d_ws;
    o.status = d_status;
    if (info.split > 1) { /* a split call with a norm waits on its partners: no status, no call */
      o.status = NULL;
      expect(arfuse_rmsnorm_ex((const void* const*)d_parts, n, d_res, d_gamma, eps, d_out, d_rout,
                               d_codes, d_scales, t, d, stream, &o) == ARFUSE_ERR_INVALID_ARG,
             "split call without a status word rejected");
      o.status = d_status;
    }
    o.fp8_out = d_fp8;
    o.fp8_inv_scale = inv_scale;
    rc = arfuse_rmsnorm_ex((const void* const*)d_parts, n, d_res, d_gamma, eps, d_out, d_rout, d_codes,
                           d_scales, t, d, stream, &o);
    if (rc == ARFUSE_OK)  /* the workspace carries over to the next call */
      rc = arfuse_rmsnorm_ex((const void* const*)d_parts, n, d_res, d_gamma, eps, d_out, d_rout,
                             d_codes, d_scales, t, d, stream, &o);
  } else if (fp8) {
    arfuse_opts o;
    memset(&o, 0, sizeof o);
    o.fp8_out = d_fp8;
    o.fp8_inv_scale = inv_scale;
    rc = arfuse_rmsnorm_ex((const void* const*)d_parts, n, d_res, d_gamma, eps, d_out, d_rout, NULL,
                           NULL, t, d, stream, &o);
  } else {
    rc = arfuse_rmsnorm((const void* const*)d_parts, n, d_res, d_gamma, eps, d_out, d_rout, d_codes,
                        d_scales, t, d, stream);
  }
  if (rc != ARFUSE_OK) fprintf(stderr, "[c-demo] call returned %d (%s)\n", rc, arfuse_status_string(rc));
  expect(rc == ARFUSE_OK, "fused call accepted");
  CHECK_HIP(hipStreamSynchronize(stream));

  uint16_t* g_out = malloc((size_t)e * 2);
  uint16_t* g_rout = malloc((size_t)e * 2);
  uint8_t* g_codes = fp4 ? malloc((size_t)e / 2) : NULL;
  uint8_t* g_scales = fp4 ? malloc((size_t)e / 16) : NULL;
  uint8_t* g_fp8 = fp8 ? malloc((size_t)e) : NULL;
  CHECK_HIP(hipMemcpy(g_out, d_out, (size_t)e * 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(g_rout, d_rout, (size_t)e * 2, hipMemcpyDeviceToHost));
  if (fp4) {
    CHECK_HIP(hipMemcpy(g_codes, d_codes, (size_t)e / 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(g_scales, d_scales, (size_t)e / 16, hipMemcpyDeviceToHost));
  }
  if (fp8) CHECK_HIP(hipMemcpy(g_fp8, d_fp8, (size_t)e, hipMemcpyDeviceToHost));
  if (d_status) {
    arfuse_ll_status h_status;
    CHECK_HIP(hipMemcpy(&h_status, d_status, sizeof h_status, hipMemcpyDeviceToHost));
    expect(h_status.code == 0 && h_status.exchange_timeouts == 0 && h_status.bad_words == 0,
           "status word clean");
  }

  /* the oracle on the same inputs */
  const uint16_t* parts[8];
  for (int i = 0; i < n; ++i) parts[i] = h_parts + i * e;
  uint16_t* w_rout = malloc((size_t)e * 2);
  uint16_t* w_out = malloc((size_t)e * 2);
  float* w_y = malloc((size_t)e * 4);
  uint8_t* w_codes = fp4 ? malloc((size_t)e / 2) : NULL;
  uint8_t* w_scales = fp4 ? malloc((size_t)e / 16) : NULL;
  uint8_t* w_fp8 = fp8 ? malloc((size_t)e) : NULL;
  expect(oracle_fused(parts, n, h_res, h_gamma, eps, t, d, w_rout, w_y, w_out, w_codes, w_scales, w_fp8,
                      inv_scale) == 0,
         "oracle accepted");

  int64_t rout_bad = 0, y_bad = 0, code_bad = 0, scale_bad = 0, fp8_bad = 0;
  for (int64_t i = 0; i < e; ++i) {
    rout_bad += g_rout[i] != w_rout[i];
    const float gy = oracle_bf16_to_f32(g_out[i]);
    y_bad += !(fabsf(gy - w_y[i]) <= 1.6e-2f + 8e-3f * fabsf(w_y[i]));
  }
  if (fp4) {
    for (int64_t i = 0; i < e / 2; ++i) code_bad += g_codes[i] != w_codes[i];
    for (int64_t i = 0; i < e / 16; ++i) scale_bad += g_scales[i] != w_scales[i];
  }
  if (fp8)
    for (int64_t i = 0; i < e; ++i) fp8_bad += g_fp8[i] != w_fp8[i];
  printf("[c-demo] n=%d t=%lld d=%lld%s%s: residual_out mismatches %lld, y out of tolerance %lld, "
         "fp4 code bytes differing %lld, scales %lld, fp8 codes %lld\n",
         n, (long long)t, (long long)d, fp4 ? " +fp4" : "", fp8 ? " +fp8" : "", (long long)rout_bad,
         (long long)y_bad, (long long)code_bad, (long long)scale_bad, (long long)fp8_bad);
  expect(rout_bad == 0, "residual_out bit-exact");
  expect(y_bad == 0, "y within tolerance");
  expect(code_bad <= 1 && scale_bad == 0, "FP4 codes and scales");
  expect(fp8_bad <= 1, "FP8 codes");

  for (int i = 0; i < n; ++i) CHECK_HIP(hipFree(d_parts[i]));
  CHECK_HIP(hipFree(d_res));
  CHECK_HIP(hipFree(d_gamma));
  CHECK_HIP(hipFree(d_out));
  CHECK_HIP(hipFree(d_rout));
  if (fp4) {
    CHECK_HIP(hipFree(d_codes));
    CHECK_HIP(hipFree(d_scales));
  }
  if (fp8) CHECK_HIP(hipFree(d_fp8));
  if (d_ws) CHECK_HIP(hipFree(d_ws));
  if (d_status) CHECK_HIP(hipFree(d_status));
  free(h_parts);
  free(h_res);
  free(h_gamma);
  free(g_out);
  free(g_rout);
  free(g_codes);
  free(g_scales);
  free(g_fp8);
  free(w_rout);
  free(w_out);
  free(w_y);
  free(w_codes);
  free(w_scales);
  free(w_fp8);
}

int main(void) {
  printf("[c-demo] library version %d\n", arfuse_version());
  fflush(stdout);
  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));

  /* argument errors: rejected synchronously, nothing enqueued */
  void* dummy[1] = {NULL};
  expect(arfuse_rmsnorm((const void* const*)dummy, 1, NULL, NULL, 1e-5f, NULL, NULL, NULL, NULL, 4,
                        1000, stream) == ARFUSE_ERR_INVALID_ARG,
         "d not a multiple of 16 rejected");
  expect(arfuse_rmsnorm((const void* const*)dummy, 9, NULL, NULL, 1e-5f, NULL, NULL, NULL, NULL, 4,
                        1024, stream) == ARFUSE_ERR_INVALID_ARG,
         "nine partials rejected");
  expect(strlen(arfuse_status_string(ARFUSE_ERR_INVALID_ARG)) > 0, "status string");

  run_case(4, 3, 1040, ARFUSE_EPI_BF16 | ARFUSE_EPI_FP4, 11, stream, 0);
  run_case(8, 2, 8192, ARFUSE_EPI_BF16 | ARFUSE_EPI_FP8, 29, stream, 0);
  run_case(8, 8, 8192, ARFUSE_EPI_BF16 | ARFUSE_EPI_FP4, 37, stream, 1);

  CHECK_HIP(hipStreamDestroy(stream));
  if (failures) {
    fprintf(stderr, "[c-demo] %d check(s) failed\n", failures);
    return 1;
  }
  printf("[c-demo] ok\n");
  return 0;
}
