/*
 * CPU oracle for the fused all-reduce epilogue: rank-ordered sum of N
 * partials, residual add, RMSNorm, optional FP4 (E2M1 + E4M3 block scale).
 *
 * TEST INFRASTRUCTURE ONLY. This header and arfuse_oracle.c are consumed by
 * the tests, by the smoke check and by the benchmark's CPU baseline. They
 * share no code with the GPU library and must never be linked into it.
 *
 * All pointers are host pointers. bf16 tensors are passed as uint16_t bit
 * patterns, row-major [t][d]. Every function is plain, scalar and slow by
 * design: it follows the definition, not a fast algorithm.
 */
#ifndef ARFUSE_ORACLE_H
#define ARFUSE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* bf16 -> fp32: exact widening (bf16 is the top half of an fp32). */
float oracle_bf16_to_f32(uint16_t b);

/* fp32 -> bf16, round to nearest, ties to the even bf16. NaN -> quiet NaN. */
uint16_t oracle_bf16_rne(float x);
void oracle_bf16_rne_array(const float* x, int64_t n, uint16_t* out);

/* OCP FP8 E4M3 ("E4M3FN": bias 7, 3 mantissa bits, max 448, no infinity).
 * value: decode a code byte. rne: nearest code to x >= 0, ties to the even
 * code; values above 448 give 448 (nearest finite value); NaN gives 0x7F. */
double oracle_e4m3_value(uint8_t code);
uint8_t oracle_e4m3_rne(float x);
void oracle_e4m3_rne_array(const float* x, int64_t n, uint8_t* out);

/* FP4 E2M1 magnitude code (0..7) of q >= 0: nearest of
 * {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even code, so above 6 gives 6. */
double oracle_e2m1_value(uint8_t mag_code);
uint8_t oracle_e2m1_rne(float q);
void oracle_e2m1_rne_array(const float* q, int64_t n, uint8_t* out);

/* Block-scaled FP4 quantization of fp32 y [t][d] (d % 16 == 0).
 * codes: uint8 [t][d/2], element 2k in the low nibble, 2k+1 in the high one.
 * scales: uint8 [t][d/16], E4M3 code of s = e4m3(blockmax / 6). */
void oracle_quantize_fp4(const float* y, int64_t t, int64_t d,
                         uint8_t* codes, uint8_t* scales);

/* The fused call. partials: host array of n pointers to bf16 [t][d].
 * Outputs (any may be NULL to skip it):
 *   residual_out bf16 [t][d]   bf16(sum_i p_i (rank order, fp32) + residual)
 *   y32          fp32 [t][d]   RMSNorm(h) * gamma before output rounding
 *   out          bf16 [t][d]   bf16(y32)
 *   codes/scales FP4 of y32 (both or neither)
 * Returns 0, or -1 on a bad argument. */
int oracle_allreduce_rmsnorm(const uint16_t* const* partials, int n,
                             const uint16_t* residual, const float* gamma,
                             float eps, int64_t t, int64_t d,
                             uint16_t* residual_out, float* y32, uint16_t* out,
                             uint8_t* codes, uint8_t* scales);

/* Step 1-3 only, exposed for the order probes: h in fp32 [t][d]. */
int oracle_rank_sum_residual(const uint16_t* const* partials, int n,
                             const uint16_t* residual, int64_t t, int64_t d,
                             float* h);

/* RMSNorm of fp32 rows h [t][d] with gamma: y32 = (h * inv) * gamma,
 * inv = 1 / sqrt(mean(h^2) + eps), fp64 inside. */
int oracle_rmsnorm_rows(const float* h, const float* gamma, float eps,
                        int64_t t, int64_t d, float* y32);

/* FP8 E4M3 of fp32 y [t][d] with a per-tensor reciprocal scale:
 * code = sign(y) << 7 | E4M3(|fl32(y * inv_scale)|), magnitudes above 448
 * giving 448. out: uint8 [t][d]. */
void oracle_quantize_fp8(const float* y, int64_t t, int64_t d, float inv_scale, uint8_t* out);

/* The fused call with every pattern: residual may be NULL (no residual add);
 * gamma may be NULL (no RMSNorm: only residual_out = bf16(h) is produced).
 * fp8_out (uint8 [t][d], may be NULL) quantizes y32 with inv_scale.
 * Returns 0, or -1 on a bad argument. */
int oracle_fused(const uint16_t* const* partials, int n, const uint16_t* residual,
                 const float* gamma, float eps, int64_t t, int64_t d,
                 uint16_t* residual_out, float* y32, uint16_t* out, uint8_t* codes,
                 uint8_t* scales, uint8_t* fp8_out, float fp8_inv_scale);

/* Sentinel-mode arrival check of one partial: the number of 16-byte vectors
 * (8 consecutive bf16 elements, n_elems % 8 == 0) holding the 16-bit sentinel
 * pattern in at least one element, i.e. not yet fully written. */
int64_t oracle_sentinel_pending(const uint16_t* part, int64_t n_elems, uint16_t sentinel);

/* LL decode of one partial: words is uint8 [n_elems/4][16] (4 bf16 payload
 * elements then a uint64 flag per 16-byte word). Writes the payload to out
 * (bf16 [n_elems]) and returns how many words carry a flag other than
 * expected_flag. */
int64_t oracle_ll_unpack(const uint8_t* words, int64_t n_elems,
                         uint64_t expected_flag, uint16_t* out);

#ifdef __cplusplus
}
#endif
#endif
