/*
 * CPU oracle for the fused all-reduce epilogue (see arfuse_oracle.h).
 *
 * TEST INFRASTRUCTURE ONLY: used by tests/, by the smoke check and by the
 * benchmark's CPU-baseline leg. It shares no code with the GPU library.
 *
 * Build: plain C99, no fast-math, no FP contraction (so that every ⊕ below is
 * one IEEE binary32 addition rounded to nearest even):
 *   gcc -O2 -std=c99 -ffp-contract=off -fno-fast-math -fPIC -shared
 *
 * What it computes, and where the pages state it:
 *  - The all-reduce result is the element-wise sum of the N rank partials,
 *    Z = sum_i Z_i ("Optimizing Tensor Parallelism Communication Overhead ...",
 *    "The Anatomy of the Tensor Parallelism Bottleneck"; "Deep Dive: AllReduce
 *    and AllReduce Fusion in TensorRT-LLM", §2.1.1).
 *  - The sum is taken in one fixed rank order so that every rank obtains the
 *    same bits ("Collectives, topology, custom all-reduce", the one-shot
 *    kernel walk-through and the determinism section), accumulated in fp32
 *    (the fp32-accumulation option, Deep Dive §3.1.5 and the FlashInfer call in
 *    "Collectives, topology, custom all-reduce").
 *  - After the sum the fused operator adds the residual, stores the new
 *    residual, applies RMSNorm with the gamma weight, stores the normalized
 *    output and optionally quantizes it (Deep Dive §6.3, the FusedOp body, and
 *    §6.5).
 *  - The FP4 format (E2M1 codes, one E4M3 scale per 16 elements, scale =
 *    block max / 6) is the workload's definition; the pages only name NVFP4.
 *
 * Parity pins for every function are in tests/test_oracle_*.py.
 */
#include "arfuse_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- bit casts */

static uint32_t f32_bits(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  return u;
}

static float bits_f32(uint32_t u) {
  float x;
  memcpy(&x, &u, 4);
  return x;
}

/* --------------------------------------------------------------------- bf16 */

float oracle_bf16_to_f32(uint16_t b) { return bits_f32((uint32_t)b << 16); }

/* Nearest bf16 to x. The two candidates are the bf16 values that bracket x:
 * "lo" = x with its low 16 bits cleared (toward zero) and "hi" = the next
 * bf16 away from zero. Their distances to x are exact in double. On a tie
 * the candidate whose last kept mantissa bit is 0 wins. A result beyond the
 * largest finite bf16 is infinity (IEEE overflow of round-to-nearest). */
uint16_t oracle_bf16_rne(float x) {
  if (isnan(x)) return (uint16_t)((f32_bits(x) >> 16) | 0x0040u);
  uint32_t u = f32_bits(x);
  uint32_t sign = u & 0x80000000u;
  uint32_t mag = u & 0x7FFFFFFFu;
  if (mag == 0x7F800000u) return (uint16_t)(u >> 16); /* infinity */
  uint32_t lo = mag & 0xFFFF0000u;
  uint32_t hi = lo + 0x10000u;
  double ax = fabs((double)x);
  double vlo = (double)bits_f32(lo);
  /* hi == 0x7F800000 is the value 2^128 in an unbounded exponent range */
  double vhi = (hi == 0x7F800000u) ? ldexp(1.0, 128) : (double)bits_f32(hi);
  double dlo = ax - vlo;
  double dhi = vhi - ax;
  uint32_t pick;
  if (dlo < dhi)
    pick = lo;
  else if (dhi < dlo)
    pick = hi;
  else
    pick = ((lo >> 16) & 1u) ? hi : lo;
  return (uint16_t)((sign | pick) >> 16);
}

void oracle_bf16_rne_array(const float* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_rne(x[i]);
}

/* --------------------------------------------------------------- FP8 E4M3 */

/* code = s eeee mmm; exponent field 0 is subnormal: m/8 * 2^-6;
 * otherwise (1 + m/8) * 2^(e-7). 0x7F / 0xFF are NaN. */
double oracle_e4m3_value(uint8_t code) {
  int s = code >> 7;
  int e = (code >> 3) & 0xF;
  int m = code & 7;
  if (e == 0xF && m == 7) return NAN;
  double v = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* Nearest non-negative finite E4M3 value by scanning all of them (codes 0x00
 * to 0x7E in increasing value). |x - v| is exact in double because both are
 * binary32 numbers. Equal distance: the even code wins. Anything above 448 is
 * nearest to 448 itself, so the scan saturates without a special case. */
uint8_t oracle_e4m3_rne(float x) {
  if (isnan(x)) return 0x7F;
  double ax = (double)x;
  if (ax < 0) ax = -ax;
  /* 448 is the largest finite code: every larger magnitude (inf included) is
   * nearer to it than to any other. Decided here because for |x| beyond
   * about 2^53 the distances below are no longer exact in double. */
  if (ax > 448.0) return 0x7E;
  uint8_t best = 0;
  double bestd = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    double dist = fabs(ax - oracle_e4m3_value((uint8_t)c));
    if (dist < bestd || (dist == bestd && (c & 1) == 0 && (best & 1) == 1)) {
      best = (uint8_t)c;
      bestd = dist;
    }
  }
  return best;
}

void oracle_e4m3_rne_array(const float* x, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_rne(x[i]);
}

/* --------------------------------------------------------------- FP4 E2M1 */

/* Magnitude codes 0..7 = exponent(2 bits) mantissa(1 bit), bias 1:
 * 0, 0.5 (subnormal), 1, 1.5, 2, 3, 4, 6. */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double oracle_e2m1_value(uint8_t mag_code) { return kE2M1[mag_code & 7]; }

uint8_t oracle_e2m1_rne(float q) {
  double aq = fabs((double)q);
  /* 6 is the largest magnitude: every larger q (inf included) is nearer to
   * it than to any other. Decided here because for q beyond about 2^55 the
   * distances below are no longer exact in double (they all round to q). */
  if (aq > 6.0) return 7;
  uint8_t best = 0;
  double bestd = INFINITY;
  for (int c = 0; c < 8; ++c) {
    double dist = fabs(aq - kE2M1[c]);
    if (dist < bestd || (dist == bestd && (c & 1) == 0 && (best & 1) == 1)) {
      best = (uint8_t)c;
      bestd = dist;
    }
  }
  return best;
}

void oracle_e2m1_rne_array(const float* q, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e2m1_rne(q[i]);
}

/* ------------------------------------------------------------ FP4 blocks */

/* One block of 16 fp32 values:
 *   bm = max |y_j|                    (exact)
 *   s  = E4M3(bm / 6)                 (fp32 division, then nearest E4M3)
 *   q_j = |y_j| / s                   (fp32 division)
 *   code_j = sign(y_j) << 3 | E2M1(q_j), magnitude 0 when s == 0. */
static void quantize_block16(const float* y, uint8_t* code16, uint8_t* scale) {
  float bm = 0.0f;
  for (int j = 0; j < 16; ++j) {
    float a = fabsf(y[j]);
    if (a > bm) bm = a;
  }
  float ratio = bm / 6.0f;
  uint8_t sc = oracle_e4m3_rne(ratio);
  float s = (float)oracle_e4m3_value(sc);
  *scale = sc;
  for (int j = 0; j < 16; ++j) {
    uint8_t mag = 0;
    if (s != 0.0f) mag = oracle_e2m1_rne(fabsf(y[j]) / s);
    code16[j] = (uint8_t)((signbit(y[j]) ? 8u : 0u) | mag);
  }
}

void oracle_quantize_fp4(const float* y, int64_t t, int64_t d, uint8_t* codes,
                         uint8_t* scales) {
  if (d % 16) return;
  uint8_t c16[16];
  for (int64_t r = 0; r < t; ++r) {
    for (int64_t b = 0; b < d / 16; ++b) {
      quantize_block16(y + r * d + b * 16, c16, scales + r * (d / 16) + b);
      for (int k = 0; k < 8; ++k)
        codes[r * (d / 2) + b * 8 + k] = (uint8_t)(c16[2 * k] | (c16[2 * k + 1] << 4));
    }
  }
}

/* ------------------------------------------------------------ FP8 output */

/* Per-tensor FP8: q = fl32(y * inv_scale) (one IEEE multiply), then the
 * nearest E4M3 magnitude (saturating at 448) with y's sign bit. */
void oracle_quantize_fp8(const float* y, int64_t t, int64_t d, float inv_scale, uint8_t* out) {
  for (int64_t e = 0; e < t * d; ++e) {
    float q = y[e] * inv_scale;
    out[e] = (uint8_t)((signbit(q) ? 0x80u : 0u) | oracle_e4m3_rne(fabsf(q)));
  }
}

/* ------------------------------------------------- sum, residual, RMSNorm */

/* acc = f32(p_0); acc = acc ⊕ f32(p_i) for i = 1..N-1; h = acc ⊕ f32(res).
 * Starting from p_0 (not from +0.0) keeps the sign of an all -0.0 sum. */
int oracle_rank_sum_residual(const uint16_t* const* partials, int n,
                             const uint16_t* residual, int64_t t, int64_t d,
                             float* h) {
  if (n < 1 || t < 0 || d < 0 || !partials || !residual || !h) return -1;
  for (int64_t e = 0; e < t * d; ++e) {
    float acc = oracle_bf16_to_f32(partials[0][e]);
    for (int i = 1; i < n; ++i) acc = acc + oracle_bf16_to_f32(partials[i][e]);
    h[e] = acc + oracle_bf16_to_f32(residual[e]);
  }
  return 0;
}

/* y_j = h_j / sqrt(mean_j(h^2) + eps) * gamma_j per row, in double:
 * ms = (sum_j h_j^2) / d (sequential sum), inv = 1 / sqrt(ms + eps),
 * y_j = (h_j * inv) * gamma_j, rounded once to fp32. */
int oracle_rmsnorm_rows(const float* h, const float* gamma, float eps, int64_t t,
                        int64_t d, float* y32) {
  if (t < 0 || d <= 0 || !h || !gamma || !y32) return -1;
  for (int64_t r = 0; r < t; ++r) {
    const float* hr = h + r * d;
    double ss = 0.0;
    for (int64_t j = 0; j < d; ++j) ss += (double)hr[j] * (double)hr[j];
    double ms = ss / (double)d;
    double inv = 1.0 / sqrt(ms + (double)eps);
    for (int64_t j = 0; j < d; ++j)
      y32[r * d + j] = (float)(((double)hr[j] * inv) * (double)gamma[j]);
  }
  return 0;
}

int oracle_allreduce_rmsnorm(const uint16_t* const* partials, int n,
                             const uint16_t* residual, const float* gamma,
                             float eps, int64_t t, int64_t d,
                             uint16_t* residual_out, float* y32, uint16_t* out,
                             uint8_t* codes, uint8_t* scales) {
  if (!residual || !gamma) return -1;
  return oracle_fused(partials, n, residual, gamma, eps, t, d, residual_out, y32, out, codes,
                      scales, NULL, 1.0f);
}

/* Every pattern of the fused operator (Deep Dive §6.3, pattern table): with
 * a residual, h = sum + residual, else h = sum; with gamma, RMSNorm and the
 * requested outputs, else only residual_out = bf16(h) (the all-reduce). */
int oracle_fused(const uint16_t* const* partials, int n, const uint16_t* residual,
                 const float* gamma, float eps, int64_t t, int64_t d,
                 uint16_t* residual_out, float* y32, uint16_t* out, uint8_t* codes,
                 uint8_t* scales, uint8_t* fp8_out, float fp8_inv_scale) {
  if (n < 1 || t < 0 || d <= 0 || !partials) return -1;
  if (!gamma && (y32 || out || codes || fp8_out)) return -1;
  if ((codes == NULL) != (scales == NULL)) return -1;
  if (codes && d % 16) return -1;
  for (int i = 0; i < n; ++i)
    if (!partials[i]) return -1;
  float* h = (float*)malloc(sizeof(float) * (size_t)d);
  float* y = (float*)malloc(sizeof(float) * (size_t)d);
  const uint16_t** prow = (const uint16_t**)malloc(sizeof(uint16_t*) * (size_t)n);
  if (!h || !y || !prow) {
    free(h);
    free(y);
    free(prow);
    return -1;
  }
  for (int64_t r = 0; r < t; ++r) {
    /* one row at a time keeps the working set small; the arithmetic is the
     * same element-wise definition as oracle_rank_sum_residual */
    for (int i = 0; i < n; ++i) prow[i] = partials[i] + r * d;
    if (residual) {
      oracle_rank_sum_residual(prow, n, residual + r * d, 1, d, h);
    } else {
      for (int64_t j = 0; j < d; ++j) {
        float acc = oracle_bf16_to_f32(prow[0][j]);
        for (int i = 1; i < n; ++i) acc = acc + oracle_bf16_to_f32(prow[i][j]);
        h[j] = acc;
      }
    }
    if (residual_out)
      for (int64_t j = 0; j < d; ++j) residual_out[r * d + j] = oracle_bf16_rne(h[j]);
    if (!gamma) continue;
    oracle_rmsnorm_rows(h, gamma, eps, 1, d, y);
    if (y32) memcpy(y32 + r * d, y, sizeof(float) * (size_t)d);
    if (out)
      for (int64_t j = 0; j < d; ++j) out[r * d + j] = oracle_bf16_rne(y[j]);
    if (codes) oracle_quantize_fp4(y, 1, d, codes + r * (d / 2), scales + r * (d / 16));
    if (fp8_out) oracle_quantize_fp8(y, 1, d, fp8_inv_scale, fp8_out + r * d);
  }
  free(h);
  free(y);
  free(prow);
  return 0;
}

/* ------------------------------------------------------------ sentinel */

int64_t oracle_sentinel_pending(const uint16_t* part, int64_t n_elems, uint16_t sentinel) {
  if (!part || n_elems < 0 || n_elems % 8) return -1;
  int64_t pending = 0;
  for (int64_t v = 0; v < n_elems / 8; ++v) {
    int hit = 0;
    for (int k = 0; k < 8; ++k) hit |= part[8 * v + k] == sentinel;
    pending += hit;
  }
  return pending;
}

/* ----------------------------------------------------------------- LL words */

int64_t oracle_ll_unpack(const uint8_t* words, int64_t n_elems,
                         uint64_t expected_flag, uint16_t* out) {
  if (!words || n_elems < 0 || n_elems % 4) return -1;
  int64_t bad = 0;
  for (int64_t w = 0; w < n_elems / 4; ++w) {
    const uint8_t* p = words + 16 * w;
    for (int k = 0; k < 4; ++k)
      out[4 * w + k] = (uint16_t)(p[2 * k] | ((uint16_t)p[2 * k + 1] << 8));
    uint64_t flag = 0;
    for (int k = 7; k >= 0; --k) flag = (flag << 8) | p[8 + k];
    if (flag != expected_flag) ++bad;
  }
  return bad;
}
