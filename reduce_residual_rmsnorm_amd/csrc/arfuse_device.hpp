// arfuse device code shared by the translation units of libarfuse.so:
// argument block, bf16/FP4/FP8/LL/sentinel helpers and the row kernel
// template. Row-kernel instances are compiled per rank count
// (arfuse_rows.hip, one object per N) so the build runs in parallel.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "arfuse.h"

namespace arfuse_detail {


typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxBlock = 1024;
constexpr int kWave = 64;

struct RowArgs {
  const u32x4* part[ARFUSE_MAX_PARTIALS];  // plain: 16 B = 8 bf16; LL: 16 B words
  u32x4* reset[ARFUSE_MAX_PARTIALS];       // sentinel layout: slots to refill
  const u32x4* residual;                   // NULL: no residual (flag kHasResidual)
  const f32x4* gamma;
  u32x4* out;
  u32x4* residual_out;                     // NULL: not written (kHasResidualOut)
  uint32_t* codes;   // 8 E2M1 codes per dword
  uint8_t* scales;
  uint8_t* fp8;      // one E4M3 code per element
  arfuse_ll_status* status;
  int64_t d8;        // 16-byte bf16 vectors per row (d / 8)
  uint64_t ll_flag;
  double inv_d;      // 1 / d (the mean's divisor), rounded once on the host
  float eps;
  float fp8_inv_scale;
  uint32_t max_polls;
  uint32_t sentinel2;  // sentinel pattern in both halves of a dword
  uint32_t flags;      // kHasResidual | kHasResidualOut | kReset
  // sentinel layout, reset by extra blocks (few rows): blocks at and past
  // `rows` each refill one block-sized chunk of one slot plane
  uint32_t rows;        // t
  uint32_t plane_vecs;  // 16-byte vectors per slot plane (t * d / 8)
  uint32_t reset_bpp;   // reset blocks per plane (plane_vecs / block, rounded up)
  // split rows: the launch has prows = rows rounded up to a multiple of 8
  // row positions per slice; workgroup b < prows << split_log2 takes column
  // slice j mod S of row 8 (j / S) + b mod 8, with j = b / 8 and S the
  // split (rows past `rows` are padding and exit), so a row's workgroups
  // share b mod 8, i.e. one XCD. They exchange their
  // sums of squares through ws: two regions of prows 128-byte lines, line r
  // holding row r's slots (slot = {fp64 share, 64-bit token of the
  // dispatch}), the first written and read through the L2, the second
  // written through to memory
  uint32_t split_log2;  // 0: one workgroup per row
  uint32_t ds8;         // 16-byte vectors per slice (d8 >> split_log2)
  u32x4* ws;
  uint32_t prows;       // split rows: rows rounded up to a multiple of 8
};

// RowArgs.flags. These features do not change the kernel's shape, so they are
// workgroup-uniform runtime branches rather than more template instances. (The
// sentinel check is a template parameter instead: its compares would otherwise
// sit in every plain instance.)
constexpr uint32_t kHasResidual = 1u;
constexpr uint32_t kHasResidualOut = 2u;
constexpr uint32_t kReset = 8u;      // sentinel layout: each row block refills its row of a.reset[]

// Epilogue mask (template parameter EPI): ARFUSE_EPI_BF16 | _FP4 | _FP8;
// 0 = no RMSNorm, the all-reduce alone.

// ------------------------------------------------------------ bf16 helpers

__device__ __forceinline__ void widen8(u32x4 r, float f[8]) {
  f[0] = __uint_as_float(r.x << 16);
  f[1] = __uint_as_float(r.x & 0xFFFF0000u);
  f[2] = __uint_as_float(r.y << 16);
  f[3] = __uint_as_float(r.y & 0xFFFF0000u);
  f[4] = __uint_as_float(r.z << 16);
  f[5] = __uint_as_float(r.z & 0xFFFF0000u);
  f[6] = __uint_as_float(r.w << 16);
  f[7] = __uint_as_float(r.w & 0xFFFF0000u);
}

// Two fp32 -> two bf16, round to nearest even: gfx950's packed conversion
// (v_cvt_pk_bf16_f32), one instruction per pair. Its rounding is checked
// against the oracle on every tie and near-tie pattern of every 16-bit prefix
// through arfuse_round_bf16.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ u32x4 narrow8(const float f[8]) {
  return u32x4{pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]),
               pack_bf16(f[6], f[7])};
}

// ------------------------------------------------------------- FP4 helpers

// The FP4 block scale: the E4M3 code of x >= 0 (OCP, bias 7, max 448),
// nearest with ties to even, and its value. gfx950's FP8 conversions do
// both: the same OCP E4M3 conversion the FP8 output takes (checked against
// the oracle on every tie pattern), after a clamp to 448 so that larger
// values saturate, and the matching decode. A bit recipe took about fifteen
// instructions for the pair.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(x, 448.0f), 0.0f, 0, false) & 0xFFu;
}

// fl32(x / 6) for the block scale, without the division sequence: x times
// fl32(1/6), corrected once by a fused multiply-add of the exact remainder
// x - 6 q0. It equals the IEEE quotient for every finite x >= 6 * 2^-126
// (an exhaustive CPU test over every binary32 pattern); below that both are
// under 2^-126, far under half the smallest E4M3 step (2^-10), so the scale
// code is 0 either way. The division sequence was about ten dependent
// instructions per lane.
__device__ __forceinline__ float div6(float x) {
  constexpr float kSixth = 1.0f / 6.0f;
  const float q0 = x * kSixth;
  return __builtin_fmaf(__builtin_fmaf(-q0, 6.0f, x), kSixth, q0);
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  return __builtin_amdgcn_cvt_f32_fp8((int)c, 0);
}

// The exact E2M1 path, taken where the hardware conversion's envelope leaves
// a decision open (see e2m1_envelope below): the magnitude code (0, .5, 1,
// 1.5, 2, 3, 4, 6 -> 0..7) of q = |y| / s, rounded to nearest with ties to
// the even code: ties at .25, 1.25, 2.5 and 5 round down, those at .75, 1.75
// and 3.5 round up, above 6 saturates.
// Instead of forming the quotient, |y| is compared with the products s*T,
// which are exact in fp32 (s has 4 significant bits, T at most 3). This takes
// the same decision as rounding the correctly rounded fp32 quotient for every
// finite |y|: the quotient's rounding can only matter within a couple of ulps
// of s*T, and an exhaustive sweep there (every scale, every threshold) finds
// no difference.
//
// The comparisons run on 16-bit keys, two elements per instruction. Each s*T
// has at most 7 significant bits, so its low 16 bits are zero and its high
// half K is exact. For a = |y| >= 0 with high half A and low half L:
//   a >= s*T  <=>  A >= K
//   a >  s*T  <=>  A + (L != 0) > K
// (A and K are at most 0x7F80, so 16-bit signed differences do not wrap.)
// s == 0 gives +inf thresholds (K = 0x7F80), which no finite |y| reaches.
struct E2M1Keys {
  // K in both 16-bit halves: the strict thresholds (ties round down) as is,
  // the others minus one (A >= K <=> K - 1 - A < 0)
  uint32_t k0, k1m1, k2, k3m1, k4, k5m1, k6;
};

__device__ __forceinline__ uint32_t rep_hi16(float t) {
  const uint32_t u = __float_as_uint(t);
  return __builtin_amdgcn_perm(u, u, 0x03020302u);  // bytes 2,3,2,3
}

__device__ __forceinline__ E2M1Keys e2m1_keys(float s) {
  const float ss = (s != 0.0f) ? s : __builtin_inff();
  const uint32_t one2 = 0x00010001u;  // no borrow between halves: every K >= 1
  return E2M1Keys{rep_hi16(ss * 0.25f), rep_hi16(ss * 0.75f) - one2, rep_hi16(ss * 1.25f),
                  rep_hi16(ss * 1.75f) - one2, rep_hi16(ss * 2.5f), rep_hi16(ss * 3.5f) - one2,
                  rep_hi16(ss * 5.0f)};
}

typedef short i16x2 __attribute__((ext_vector_type(2)));

// 0xFFFF in each half where x - y < 0 (16-bit signed), else 0: a packed
// subtract and a packed arithmetic shift. The mask is hidden from the
// optimizer, which otherwise turns each bfi() of it into a compare and a
// select per half.
__device__ __forceinline__ uint32_t lt16(uint32_t x, uint32_t y) {
  const i16x2 d = __builtin_bit_cast(i16x2, x) - __builtin_bit_cast(i16x2, y);
  uint32_t m = __builtin_bit_cast(uint32_t, (i16x2)(d >> (short)15));
  asm("" : "+v"(m));
  return m;
}

__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t x, uint32_t y) {
  return (m & x) | (~m & y);
}

// The 4-bit codes of two elements of one block: y0's in bits 0..3, y1's in
// bits 16..19 (sign in bit 3 of each). Three levels of comparison find the
// magnitude, the number of thresholds |y| passes: t3 splits {0..3} from
// {4..7}, then t1 or t5, then one of the strict ones. No branches.
__device__ __forceinline__ uint32_t e2m1_two(float y0, float y1, const E2M1Keys& k) {
  const uint32_t u0 = __float_as_uint(y0), u1 = __float_as_uint(y1);
  const uint32_t hi = __builtin_amdgcn_perm(u1, u0, 0x07060302u);  // high halves
  const uint32_t a = hi & 0x7FFF7FFFu;
  // A + (L != 0): the high half of u + 0xFFFF (no carry reaches the sign:
  // the exponent of a finite value is below 0xFF)
  const uint32_t ac =
      __builtin_amdgcn_perm(u1 + 0xFFFFu, u0 + 0xFFFFu, 0x07060302u) & 0x7FFF7FFFu;
  const uint32_t g2 = lt16(k.k3m1, a);                           // a >= t3
  const uint32_t g1 = lt16(bfi(g2, k.k5m1, k.k1m1), a);          // a >= t5 or t1
  const uint32_t tl = bfi(g2, bfi(g1, k.k6, k.k4), bfi(g1, k.k2, k.k0));
  const uint32_t g0 = lt16(tl, ac);                              // a > t6, t4, t2 or t0
  return (g0 & 0x00010001u) | (g1 & 0x00020002u) | (g2 & 0x00040004u) |
         ((hi >> 12) & 0x00080008u);
}

// Value of lane (lane XOR 1) for CTRL = 0xB1 (quad_perm [1,0,3,2]), of lane
// (lane XOR 2) for CTRL = 0x4E (quad_perm [2,3,0,1]): a DPP move, a plain
// vector instruction (a wave shuffle would go through the LDS unit).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Fast E2M1 codes by gfx950's FP4 conversion, exact by an envelope.
// v_cvt_scalef32_pk_fp4_f32 with scale 1 rounds an fp32 value to E2M1 to
// nearest even, saturating at 6, sign kept (-0 and negatives that round to 0
// give 0x8), src0 in the low nibble: a GPU probe over every value within
// 2048 ulps of each E2M1 value and decision point, both signs, specials and
// 200,000 random values found no difference from the oracle's rounding. The
// oracle rounds q = fl32(|y| / s); here each y is multiplied by r_lo and
// r_hi, the hardware reciprocal of s moved 2^-20 down and up. The
// reciprocal is within 1 ulp and each product rounds once, so
// |fl(y r_lo)| <= |fl32(y / s)| <= |fl(y r_hi)|; the rounding is monotone in
// |q|, so where the two conversions agree they give the oracle's code. s = 0
// takes r = 0: every magnitude 0, sign kept, as the oracle rules. Where they
// differ (q within about 2^-20 of a decision point: rare), the lane takes
// the exact comparisons (e2m1_two). Against e2m1_two alone, about 30
// instructions per lane instead of about 100.
struct E2M1Envelope {
  float lo, hi;  // r_lo, r_hi
};

__device__ __forceinline__ E2M1Envelope e2m1_envelope(float s) {
  const float r = (s != 0.0f) ? __builtin_amdgcn_rcpf(s) : 0.0f;
  return E2M1Envelope{r * (1.0f - 0x1p-20f), r * (1.0f + 0x1p-20f)};
}

template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2(uint32_t old, float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// FP4 of the 8 values a lane holds. Lanes (2m, 2m+1) hold one 16-element
// block, so the block max is one lane swap (lane XOR 1) away. Every lane of the
// wave must call this (the swap reads the partner lane's register).
__device__ __forceinline__ void fp4_pair(const float y[8], uint32_t& codes8, uint32_t& scale) {
  float am = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(y[e]));
  am = fmaxf(am, dpp_f32<0xB1>(am));
  const uint32_t sc = e4m3_code(div6(am));
  const float s = e4m3_value(sc);
  const E2M1Envelope r = e2m1_envelope(s);
  uint32_t lo = 0, hi = 0;
  lo = cvt_fp4x2<0>(lo, y[0] * r.lo, y[1] * r.lo);
  hi = cvt_fp4x2<0>(hi, y[0] * r.hi, y[1] * r.hi);
  lo = cvt_fp4x2<1>(lo, y[2] * r.lo, y[3] * r.lo);
  hi = cvt_fp4x2<1>(hi, y[2] * r.hi, y[3] * r.hi);
  lo = cvt_fp4x2<2>(lo, y[4] * r.lo, y[5] * r.lo);
  hi = cvt_fp4x2<2>(hi, y[4] * r.hi, y[5] * r.hi);
  lo = cvt_fp4x2<3>(lo, y[6] * r.lo, y[7] * r.lo);
  hi = cvt_fp4x2<3>(hi, y[6] * r.hi, y[7] * r.hi);
  uint32_t c = lo;
  if (__builtin_expect(lo != hi, 0)) {
    // exact comparisons; elements m and m + 4 share a key pair, so the four
    // pairs' codes land in place with three shifts: nibble e at bits 4e
    const E2M1Keys k = e2m1_keys(s);
    c = e2m1_two(y[0], y[4], k);
#pragma unroll
    for (int m = 1; m < 4; ++m) c |= e2m1_two(y[m], y[m + 4], k) << (4 * m);
  }
  codes8 = c;
  scale = sc;
}

// ------------------------------------------------------------- LL helpers

__device__ __forceinline__ bool ll_ok(u32x4 w, uint64_t flag) {
  return (w.z == (uint32_t)flag) & (w.w == (uint32_t)(flag >> 32));
}

// Store of a 16-byte word that workgroups on other CUs poll: written through
// the caches (sc0 sc1, the same policy as reread16), one instruction, so a
// reader sees either the old word or all of the new one.
__device__ __forceinline__ void store16_through(char* base, uint32_t bytes, uint32_t off, u32x4 v);

// The re-read of a split row's exchange slot in the region its partners on
// the same XCD find in their L2. The compiler issues it exactly as reread16
// (a volatile buffer load gets sc0 sc1); its own policy immediate (sc0 and
// volatile) only keeps the two polls of the exchange loop two instructions
// the compiler does not merge: merged, split chains moved by -0.01 to
// +0.025 us per call.
constexpr int kRereadL2Policy = (int)0x80000001u;
__device__ __forceinline__ u32x4 reread16_l2(const char* row, uint32_t row_bytes, uint32_t off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)row, (short)0, (int)row_bytes, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kRereadL2Policy);
}

// Store of a 16-byte word for partners on the same XCD (sc0 only: through
// the L1 into the XCD's L2, which keeps the line instead of writing it
// through to memory).
__device__ __forceinline__ void store16_l2(char* base, uint32_t bytes, uint32_t off, u32x4 v) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0x1);
}

// Re-read of a 16-byte vector another agent may still be writing: a buffer
// load through a descriptor of the row (scalar registers) at the lane's
// 32-bit offset, bypassing the caches (sc0 sc1) and kept in the polling loop
// (the compiler's volatile bit, 1 << 31). A pointer-based volatile load would
// need a 64-bit address per partial in vector registers, and the compiler
// keeps all of them live through the row. Word 3 of the descriptor: raw
// 32-bit data format, as gfx9-family buffer resources take it.
constexpr int kRereadPolicy = (int)0x80000011u;
constexpr int kBufferWord3 = 0x00020000;
__device__ __forceinline__ u32x4 reread16(const char* row, uint32_t row_bytes, uint32_t off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)row, (short)0, (int)row_bytes, kBufferWord3);
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kRereadPolicy);
}

__device__ __forceinline__ void store16_through(char* base, uint32_t bytes, uint32_t off, u32x4 v) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, kBufferWord3);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kRereadPolicy);
}

// Split rows: bounded wait for a partner's slot (about a quarter second).
constexpr uint32_t kExchangePolls = 1u << 18;

// The dispatch id of the running kernel (an SGPR pair the command processor
// fills at wave launch: the index of the dispatch packet in its queue).
extern "C" __device__ uint64_t arfuse_llvm_dispatch_id() __asm("llvm.amdgcn.dispatch.id");

// The token a split row's slices tag their exchange slots with: one value
// per kernel dispatch. Every workgroup of a dispatch reads the same dispatch
// id, and the command processor numbers the packets of a queue in order, so
// consecutive calls and graph replays on a queue differ; queues keep their
// own counts, so the queue's address (another SGPR pair) is mixed into the
// high word. Bit 0 of the high word is set, so a zeroed slot never matches.
// A slot carrying any other token (an earlier call of any shape, another
// queue's call, garbage) reads as "not yet written": the slots need no
// clearing between calls or when the shape changes.
__device__ __forceinline__ u32x2 dispatch_token() {
  const uint64_t did = arfuse_llvm_dispatch_id();
  const uint64_t q = (uint64_t)__builtin_amdgcn_queue_ptr();
  return u32x2{(uint32_t)did,
               ((uint32_t)(q >> 12) ^ (uint32_t)(q >> 44) ^ (uint32_t)(did >> 32)) | 1u};
}

// 1 / sqrt(ss / d + eps) in fp64: the hardware reciprocal square root
// refined by two Newton steps on the residual e = 1 - x r^2 (r += r e / 2),
// each step squaring the relative error, so the result is within a few
// fp64 ulps of the correctly rounded value. The library's square root and
// division take about sixty dependent fp64 instructions, which every wave
// repeats: at four waves per SIMD that cost 0.3 us per decode call.
__device__ __forceinline__ double inv_rms(double ss, double inv_d, double eps) {
  const double x = ss * inv_d + eps;
  double r = __builtin_amdgcn_rsq(x);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const double e = __builtin_fma(-(x * r), r, 1.0);
    r = __builtin_fma(0.5 * r, e, r);
  }
  return r;
}

// A word whose flag does not match is re-read, a short sleep apart, at most
// max_polls times. Returns the last word read; *bad counts a word that never
// matched.
__device__ __forceinline__ u32x4 ll_repoll(const char* row, uint32_t row_bytes, uint32_t off,
                                           u32x4 w, uint64_t flag, uint32_t max_polls,
                                           uint32_t* bad) {
  for (uint32_t i = 0; i < max_polls; ++i) {
    __builtin_amdgcn_s_sleep(2);
    w = reread16(row, row_bytes, off);
    if (ll_ok(w, flag)) return w;
  }
  *bad += 1;
  return w;
}

// Sentinel layout: does a 16-byte vector still hold the sentinel pattern in
// any of its 8 bf16 elements? (s2 = the pattern in both halves of a dword.)
__device__ __forceinline__ bool holds_sentinel(u32x4 w, uint32_t s2) {
  const uint32_t lo = s2 & 0xFFFFu;
  const uint32_t hi = s2 & 0xFFFF0000u;
  return ((w.x & 0xFFFFu) == lo) | ((w.x & 0xFFFF0000u) == hi) | ((w.y & 0xFFFFu) == lo) |
         ((w.y & 0xFFFF0000u) == hi) | ((w.z & 0xFFFFu) == lo) | ((w.z & 0xFFFF0000u) == hi) |
         ((w.w & 0xFFFFu) == lo) | ((w.w & 0xFFFF0000u) == hi);
}

// Sentinel layout: nonzero iff some 16-bit half of the vector equals the
// pattern. Per dword t = w ^ s2, a half of t is zero
// iff (t - 0x00010001) & ~t has that half's top bit set; a borrow out of a
// zero low half can only flag the high half when the low one already is.
__device__ __forceinline__ uint32_t zero_half4(u32x4 w, uint32_t s2) {
  const uint32_t a = w.x ^ s2, b = w.y ^ s2, c = w.z ^ s2, d = w.w ^ s2;
  return (((a - 0x00010001u) & ~a) | ((b - 0x00010001u) & ~b) | ((c - 0x00010001u) & ~c) |
          ((d - 0x00010001u) & ~d)) & 0x80008000u;
}

// Re-read a vector that still holds the sentinel, bounded like ll_repoll.
__device__ __forceinline__ u32x4 sentinel_repoll(const char* row, uint32_t row_bytes,
                                                 uint32_t off, u32x4 w, uint32_t s2,
                                                 uint32_t max_polls, uint32_t* bad) {
  for (uint32_t i = 0; i < max_polls; ++i) {
    __builtin_amdgcn_s_sleep(2);
    w = reread16(row, row_bytes, off);
    if (!holds_sentinel(w, s2)) return w;
  }
  *bad += 1;
  return w;
}

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

__device__ __forceinline__ void store16(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

// DPP lane move of a double (two 32-bit halves). MOV: a plain DPP move
// (every source lane is in the row and active here, so bound_ctrl never
// applies) instead of an update of a zeroed register, which costs a v_mov
// per half per step: whole-row decode 0.04-0.08 us faster, prefill t=512
// 0.2 us. Split slices keep the update form, which measured 0.05 us faster
// for them.
template <int CTRL, bool MOV = true>
__device__ __forceinline__ double dpp_f64(double v) {
  int lo, hi;
  if constexpr (MOV) {
    lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xF, 0xF, true);
    hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xF, 0xF, true);
  } else {
    lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xF, 0xF, false);
    hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xF, 0xF, false);
  }
  return __hiloint2double(hi, lo);
}

// Sum of a double over each row of 16 lanes, in every lane of the row: quad
// swaps (lane ^ 1, lane ^ 2), then the mirror inside each half row (quad 0
// with quad 1), then the mirror inside the row (half 0 with half 1). The
// additions are commutative pairs, so every lane of a row gets the same bits.
template <bool MOV = true>
__device__ __forceinline__ double row16_sum(double v) {
  v += dpp_f64<0xB1, MOV>(v);   // quad_perm [1,0,3,2]
  v += dpp_f64<0x4E, MOV>(v);   // quad_perm [2,3,0,1]
  v += dpp_f64<0x141, MOV>(v);  // row_half_mirror
  v += dpp_f64<0x140, MOV>(v);  // row_mirror
  return v;
}

__device__ __forceinline__ double lane_f64(double v, int l) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                          __builtin_amdgcn_readlane(__double2loint(v), l));
}

// Sum over the wave's 64 lanes (same value in every lane): the four row sums
// added in row order. A fixed tree: the result does not depend on timing.
template <bool MOV = true>
__device__ __forceinline__ double wave_sum(double v) {
  v = row16_sum<MOV>(v);
  return ((lane_f64(v, 0) + lane_f64(v, 16)) + lane_f64(v, 32)) + lane_f64(v, 48);
}

// ------------------------------------------------------------- row kernel

// Lane geometry. A thread handles 8 elements of its row per chunk k < VPT, as
// two groups of 4 (j = 0, 1); group_elem() is the row offset of a group's
// first element.
//  plain: the 8 elements are the contiguous 16-byte vector v = k*nthr + lane.
//  LL: each 16-byte word carries 4 elements, so the wave's 128 words of a
//      chunk are loaded as two fully contiguous 1 KiB instructions: lane i
//      takes words i and 64 + i of the wave's tile, i.e. groups at tile
//      offsets 4i and 256 + 4i.
template <bool LL>
__device__ __forceinline__ int64_t group_elem(int k, int j, int lane, int nthr) {
  if constexpr (LL)
    return 8 * ((int64_t)k * nthr + (lane & ~(kWave - 1))) + 256 * j + 4 * (lane & (kWave - 1));
  else
    return 8 * ((int64_t)k * nthr + lane) + 4 * j;
}

template <bool NT>
__device__ __forceinline__ u32x2 load8(const u32x2* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

// FP4 of a 4-element group in the LL geometry: lanes 4m..4m+3 hold one
// 16-element block (two lane swaps give its max); 4 codes = 16 bits.
__device__ __forceinline__ void fp4_quad(const float* y, uint32_t& codes4, uint32_t& scale) {
  float am = fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fmaxf(fabsf(y[2]), fabsf(y[3])));
  am = fmaxf(am, dpp_f32<0xB1>(am));
  am = fmaxf(am, dpp_f32<0x4E>(am));
  const uint32_t sc = e4m3_code(div6(am));
  const float s = e4m3_value(sc);
  const E2M1Envelope r = e2m1_envelope(s);
  uint32_t lo = 0, hi = 0;
  lo = cvt_fp4x2<0>(lo, y[0] * r.lo, y[1] * r.lo);
  hi = cvt_fp4x2<0>(hi, y[0] * r.hi, y[1] * r.hi);
  lo = cvt_fp4x2<1>(lo, y[2] * r.lo, y[3] * r.lo);
  hi = cvt_fp4x2<1>(hi, y[2] * r.hi, y[3] * r.hi);
  uint32_t c = lo;
  if (__builtin_expect(lo != hi, 0)) {
    // exact comparisons: pairs (0, 2) and (1, 3) give nibbles 0 and 1 in
    // byte 0, 2 and 3 in byte 2
    const E2M1Keys k = e2m1_keys(s);
    const uint32_t t = e2m1_two(y[0], y[2], k) | (e2m1_two(y[1], y[3], k) << 4);
    c = __builtin_amdgcn_perm(t, t, 0x0C0C0200u);  // bytes 0, 2
  }
  codes4 = c;
  scale = sc;
}

// FP8 E4M3 codes of four values times inv_scale, packed little-endian into a
// dword: gfx950's OCP E4M3 conversion (round to nearest even, sign kept) on
// q = fl32(y * inv_scale) clamped to [-448, 448] first, so magnitudes above
// 448 saturate to 448 instead of becoming NaN.
__device__ __forceinline__ uint32_t fp8_quad(const float* y, float inv_scale) {
  float q[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) q[e] = __builtin_amdgcn_fmed3f(y[e] * inv_scale, -448.0f, 448.0f);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], r, true);
  return (uint32_t)r;
}

// Typed access at a byte offset from a base pointer. Row base pointers are
// uniform across the workgroup (scalar registers) and lane offsets fit in 32
// bits (rows are at most 65536 elements), so every load and store takes the
// scalar-base + 32-bit vector-offset form and a lane keeps one offset register
// for all N + 1 input streams instead of a 64-bit address per stream; that
// leaves room to keep all of a row's loads in flight at once.
template <typename T>
__device__ __forceinline__ const T* at(const char* base, uint32_t off) {
  return reinterpret_cast<const T*>(base + off);
}
template <typename T>
__device__ __forceinline__ T* at_w(char* base, uint32_t off) {
  return reinterpret_cast<T*>(base + off);
}

// Row output store policies. STREAM instances (chosen by the host when a
// call's rows take several rounds of workgroups: prefill) store with device
// scope (sc1) through a buffer descriptor of the row, which writes through
// to memory instead of leaving the lines to the L2: prefill N=8 t=4096
// d=8192 121.0 -> 117.2 us, the all-reduce alone 114.3 -> 109.1, d=32768
// t=1024 131 -> 122 us, on the same box; decode loses 0.25-0.45 us per call
// with these stores (the next call's reads of residual_out miss). Whole rows
// in one round of workgroups or less (decode, t=512) store with the default
// policy, into the L2, which writes the lines back as the kernel ends, and
// load the residual with the default policy too: t=512 N=8 16.9 -> 15.9-16.0
// us against non-temporal stores and loads, whole-row decode chains within
// 0.005 us. Split rows keep non-temporal stores and residual loads, 0.005-
// 0.014 us per decode call faster than the default policy. The choice is a
// template parameter: as a run-time branch it cost every decode call 0.05 us.
constexpr int kStoreNT = 0;       // non-temporal
constexpr int kStoreL2 = 1;       // default policy
constexpr int kStoreThrough = 2;  // device scope (sc1), written through
constexpr int kStreamPolicy = 0x10;  // sc1
template <int POL, typename T>
__device__ __forceinline__ void out_store(char* base, uint32_t off, T v) {
  if constexpr (POL == kStoreThrough) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7FFFFFFF, kBufferWord3);
    if constexpr (sizeof(T) == 16)
      __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kStreamPolicy);
    else if constexpr (sizeof(T) == 8)
      __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, kStreamPolicy);
    else
      __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, kStreamPolicy);
  } else if constexpr (POL == kStoreNT) {
    __builtin_nontemporal_store(v, at_w<T>(base, off));
  } else {
    *at_w<T>(base, off) = v;
  }
}

// Row-kernel variants beyond layout and epilogue: one workgroup per row with
// non-temporal output stores (decode), split rows, or one workgroup per row
// with streaming stores (prefill; see out_store).
constexpr int kRowWhole = 0;
constexpr int kRowSplit = 1;
constexpr int kRowStream = 2;

// Pipeline depth of a row kernel instance: how many chunks' loads may be in
// flight while a chunk is processed. A chunk is N partial loads (two words
// each for LL) plus the residual, 4 VGPRs per 16 bytes; h keeps 8 floats per
// chunk for the whole row. All chunks at once (D = VPT) while that fits the
// 128 VGPRs of a 1024-thread block with room to spare, else two, else one.
template <int N, int VPT, bool LL>
constexpr int pipeline_depth() {
  constexpr int chunk = 4 * N * (LL ? 2 : 1) + 4;
  constexpr int fixed = 8 * VPT + 28;
  if (VPT * chunk + 8 * VPT + fixed <= 112) return VPT;  // gamma preloaded too
  if (2 * chunk + fixed <= 112) return 2 < VPT ? 2 : VPT;
  return 1;
}

template <int N, int VPT, bool LL, bool SENT, int EPI, int KIND>
__global__ __launch_bounds__(kMaxBlock) void row_kernel(RowArgs a) {
  constexpr bool SPLIT = KIND == kRowSplit;
  constexpr bool STREAM = KIND == kRowStream;
  // output store policy, and whether the residual is loaded non-temporally
  // (see out_store)
  constexpr int SPOL = STREAM ? kStoreThrough : SPLIT ? kStoreNT : kStoreL2;
  constexpr bool RES_NT = KIND != kRowWhole;
  constexpr bool NORM = EPI != 0;
  constexpr bool OUT = (EPI & ARFUSE_EPI_BF16) != 0;
  constexpr bool FP4 = (EPI & ARFUSE_EPI_FP4) != 0;
  constexpr bool FP8 = (EPI & ARFUSE_EPI_FP8) != 0;
  constexpr int D = pipeline_depth<N, VPT, LL>();
  constexpr bool ALL_AT_ONCE = D == VPT;
  constexpr int W = LL ? 2 : 1;  // 16-byte loads per partial per chunk
  // gamma, when the whole row's loads fit at once: a split row's slice and a
  // streaming (several-round) row load it with their partials, except in
  // the sentinel layout: there a split slice loads it right after the
  // arrival check, so the re-poll path's registers stay free, and a
  // streaming row after its rank sum. A whole row in one round loads it
  // after its rank sum: gamma is not needed before the row's norm, and left
  // out of the first loads it does not share the one CU's fetch with the
  // partials (decode chains 0.03-0.1 us faster, t=512 0.45 us faster; split
  // rows, whose slices fetch little, measured 0.05-0.17 us slower that way,
  // and the timed prefill 1.2% slower). Wide rows load it per chunk in the
  // output loop.
  constexpr bool G_EARLY = NORM && ALL_AT_ONCE && (SPLIT || STREAM) && !SENT;
  constexpr bool G_AFTER_ARRIVAL = NORM && ALL_AT_ONCE && SPLIT && SENT;
  constexpr bool G_AFTER_SUM = NORM && ALL_AT_ONCE && !SPLIT && !G_EARLY;
  const int lane = threadIdx.x;
  const int nthr = blockDim.x;
  if constexpr (SPLIT) {
    // Split rows: every launch argument the row's first loads depend on, in
    // one batch of scalar loads. The arguments are in memory the scalar cache
    // has not seen; left to itself the compiler issued them in several
    // batches (the residual's branch splits them), each a memory round trip
    // before the first vector load. Measured on 160-call chains: 0.05-0.15 us
    // per call. Whole rows keep the compiler's order, which measured faster
    // for them.
    asm volatile("" ::"s"(a.part[0]), "s"(a.part[1]), "s"(a.part[2]), "s"(a.part[3]),
                 "s"(a.part[4]), "s"(a.part[5]), "s"(a.part[6]), "s"(a.part[7]), "s"(a.residual),
                 "s"(a.gamma), "s"(a.out), "s"(a.residual_out), "s"(a.d8), "s"(a.flags),
                 "s"(a.rows), "s"(a.split_log2), "s"(a.ds8), "s"(a.prows));
  }
  // split instances are launched with split_log2 >= 1; the others fold every
  // slice computation away
  const uint32_t lg = SPLIT ? a.split_log2 : 0u;
  const uint32_t prows = SPLIT ? a.prows : a.rows;  // row positions per slice
  const uint32_t row_blocks = prows << lg;
  if constexpr (SENT) {
    // a reset block (only launched when the rows are few): refill one chunk
    // of one slot plane of the set a later call reuses, a vector per lane,
    // on a CU that no row occupies
    if (blockIdx.x >= row_blocks) {
      const uint32_t b = blockIdx.x - row_blocks;
      const uint32_t i = b / a.reset_bpp;
      const uint32_t v = (b - i * a.reset_bpp) * (uint32_t)nthr + (uint32_t)lane;
      if (v < a.plane_vecs) store16(a.reset[i] + v, u32x4{a.sentinel2, a.sentinel2, a.sentinel2, a.sentinel2});
      return;
    }
  }
  // this workgroup's columns: the whole row, or one slice of a split row.
  // The workgroups of a launch go to the XCDs in turn (b mod 8), so with
  // j = b / 8 the index of b among its XCD's workgroups, b takes slice
  // j mod S of row 8 (j / S) + b mod 8: a row's slices share an XCD, and
  // its L2 for their exchange, and are consecutive there, dispatched
  // together. Shifts and masks (prows is a multiple of 8), where a modulo by
  // the runtime prows was a scalar division sequence before the first load:
  // 0.025-0.045 us per decode call with t > 8.
  const uint32_t bj = blockIdx.x >> 3;
  const uint32_t row = SPLIT ? ((bj >> lg) << 3) | (blockIdx.x & 7u) : blockIdx.x;
  const uint32_t slice = SPLIT ? bj & ((1u << lg) - 1u) : 0u;
  if constexpr (SPLIT) {
    if (row >= a.rows) return;  // padding row position
  }
  const uint32_t d = (uint32_t)(a.d8 * 8);  // the row width: the mean's divisor
  const uint32_t ds = SPLIT ? a.ds8 * 8 : d;  // the columns this workgroup handles
  const int64_t rb = (int64_t)row * d + (int64_t)slice * ds;  // its first element
  const bool has_res = (a.flags & kHasResidual) != 0;
  const bool has_rout = (a.flags & kHasResidualOut) != 0;
  // row bases: partials (bf16, or LL words of 4 bytes per element), residual,
  // outputs (bf16), FP4 codes (half a byte per element), scales (1/16), FP8
  const char* prow[N];
#pragma unroll
  for (int i = 0; i < N; ++i) prow[i] = (const char*)a.part[i] + rb * (LL ? 4 : 2);
  const char* rrow = (const char*)a.residual + rb * 2;
  const char* grow = (const char*)a.gamma + (int64_t)slice * ds * 4;
  char* orow = (char*)a.residual_out + rb * 2;
  char* yrow = (char*)a.out + rb * 2;
  char* crow = (char*)a.codes + rb / 2;
  char* srow = (char*)a.scales + rb / 16;
  char* frow = (char*)a.fp8 + rb;

  // group offsets (elements), clamped into the row for idle lanes so every
  // load stays in bounds; idle lanes store nothing and add nothing
  uint32_t eo[VPT][2];
  bool ok[VPT][2];
  auto set_offsets = [&](int k, int ln) {
    if constexpr (LL) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t e = (uint32_t)group_elem<LL>(k, j, ln, nthr);
        ok[k][j] = e < ds;
        eo[k][j] = ok[k][j] ? e : ds - 4;
      }
    } else {  // the two groups of a plain vector share one validity
      const uint32_t e = (uint32_t)group_elem<LL>(k, 0, ln, nthr);
      ok[k][0] = ok[k][1] = e < ds;
      eo[k][0] = ok[k][0] ? e : ds - 8;
      eo[k][1] = eo[k][0] + 4;
    }
  };
  // Wide rows recompute the offsets in each phase from a copy of the lane
  // index the compiler cannot see through, so one phase's offsets do not stay
  // live (in registers) through the next.
  auto fresh_offsets = [&]() {
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int k = 0; k < VPT; ++k) set_offsets(k, ln);
  };
#pragma unroll
  for (int k = 0; k < VPT; ++k) set_offsets(k, lane);

  u32x4 raw[VPT][N][W];
  u32x4 rres[VPT];
  f32x4 g[VPT][2];
  float h[VPT][8];
  uint32_t bad = 0;

  // ---- per-chunk steps. The lambdas that load take the row bases by value:
  // captured by reference, the loads lose the scalar-base + 32-bit-offset
  // form and each gets a 64-bit address in vector registers.
  auto load_gamma = [&, grow](int k) {
    g[k][0] = *at<f32x4>(grow, eo[k][0] * 4);
    g[k][1] = *at<f32x4>(grow, eo[k][1] * 4);
  };
  auto load_chunk = [&, prow, rrow](int k) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if constexpr (LL) {
        raw[k][i][0] = load16<true>(at<u32x4>(prow[i], eo[k][0] * 4));
        raw[k][i][1] = load16<true>(at<u32x4>(prow[i], eo[k][1] * 4));
      } else {
        // partial 0 with the default policy instead of non-temporal, where
        // measured faster: the all-reduce alone in a streaming row with
        // N >= 6 (t=4096, N=8: 107.3-107.6 -> 100.5-100.8 us, without
        // residual 95.5-95.7 -> 89.2-89.3; N=6: 86.4-86.8 -> 80.8-80.9),
        // and a normalizing one-round row with N = 8 (t=512: 15.80-15.91 ->
        // 15.63-15.65 us). The other cases lost: the all-reduce at N=4 (62.8-
        // 63.1 -> 68.5-68.9), normalizing one-round rows at N=6 and 4 (3-7%),
        // normalizing streaming rows (7%), and two default-policy partials
        // at t=512 (10%).
        if (i == 0 && ((STREAM && !NORM && N >= 6) || (KIND == kRowWhole && NORM && N == 8 && !SENT)))
          raw[k][i][0] = load16<false>(at<u32x4>(prow[i], eo[k][0] * 2));
        else
          raw[k][i][0] = load16<true>(at<u32x4>(prow[i], eo[k][0] * 2));
      }
    }
    rres[k] = u32x4{0, 0, 0, 0};
    if (has_res) {
      if constexpr (LL) {
        const u32x2 r0 = load8<RES_NT>(at<u32x2>(rrow, eo[k][0] * 2));
        const u32x2 r1 = load8<RES_NT>(at<u32x2>(rrow, eo[k][1] * 2));
        rres[k] = u32x4{r0.x, r0.y, r1.x, r1.y};
      } else {
        rres[k] = load16<RES_NT>(at<u32x4>(rrow, eo[k][0] * 2));
      }
    }
    if constexpr (G_EARLY) load_gamma(k);
  };
  // Arrival of chunk k. LL: the filter is the OR of (flag XOR expected) over
  // the lane's words; sentinel: a zero 16-bit half in (data XOR pattern),
  // over whole dwords. Both are vector integer ops: per-word or per-element
  // compares would each make a lane mask for the scalar unit to combine, a
  // long serial chain. Only a lane the filter flags runs the exact check and
  // the bounded re-poll.
  auto arrive = [&, prow](int k) {
    if constexpr (LL) {
      const uint32_t flo = (uint32_t)a.ll_flag, fhi = (uint32_t)(a.ll_flag >> 32);
      uint32_t mis = 0;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < N; ++i) m |= (raw[k][i][j].z ^ flo) | (raw[k][i][j].w ^ fhi);
        mis |= ok[k][j] ? m : 0u;
      }
      if (__builtin_expect(mis != 0, 0)) {
#pragma unroll
        for (int i = 0; i < N; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            if (ok[k][j] && !ll_ok(raw[k][i][j], a.ll_flag))
              raw[k][i][j] = ll_repoll(prow[i], ds * 4, eo[k][j] * 4, raw[k][i][j], a.ll_flag,
                                       a.max_polls, &bad);
      }
    } else if constexpr (SENT) {
      uint32_t z = 0;
#pragma unroll
      for (int i = 0; i < N; ++i) z |= zero_half4(raw[k][i][0], a.sentinel2);
      z = ok[k][0] ? z : 0u;
      if (__builtin_expect(z != 0, 0)) {
#pragma unroll
        for (int i = 0; i < N; ++i)
          if (ok[k][0] && holds_sentinel(raw[k][i][0], a.sentinel2))
            raw[k][i][0] = sentinel_repoll(prow[i], ds * 2, eo[k][0] * 2, raw[k][i][0],
                                           a.sentinel2, a.max_polls, &bad);
      }
    }
  };
  // rank-ordered fp32 sum of chunk k, residual last
  auto rank_sum = [&](int k) {
    u32x4 pv[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if constexpr (LL)
        pv[i] = u32x4{raw[k][i][0].x, raw[k][i][0].y, raw[k][i][1].x, raw[k][i][1].y};
      else
        pv[i] = raw[k][i][0];
    }
    float acc[8], f[8];
    widen8(pv[0], acc);
#pragma unroll
    for (int i = 1; i < N; ++i) {
      widen8(pv[i], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] + f[e];
    }
    if (has_res) {
      widen8(rres[k], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) h[k][e] = acc[e] + f[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) h[k][e] = acc[e];
    }
  };
  double ss = 0.0;
  // residual_out of chunk k
  auto store_residual = [&](int k) {
    if (has_rout) {
      const u32x4 hb = narrow8(h[k]);
      if constexpr (LL) {
        if (ok[k][0]) out_store<SPOL>(orow, eo[k][0] * 2, u32x2{hb.x, hb.y});
        if (ok[k][1]) out_store<SPOL>(orow, eo[k][1] * 2, u32x2{hb.z, hb.w});
      } else if (ok[k][0]) {
        out_store<SPOL>(orow, eo[k][0] * 2, hb);
      }
    }
  };
  // chunk k's share of the sum of squares; without a norm (except in a
  // streaming row, below), or in a split row, its residual_out.
  // A whole row that normalizes stores residual_out next to y, in the output
  // loop, so the row's two output streams reach HBM together, after its
  // reads, rather than one in the middle of them. Prefill N=8 d=8192: t=4096
  // 1-1.5% faster, t=512 1%, d=32768 2.5-3.5%; whole-row decode calls within
  // +-0.06 us either way. A split row stores it here, before the exchange,
  // whose wait the stores then overlap: 160-call chains 0.03-0.12 us faster
  // (FP4 t=64 3.24 -> 3.17 us, N=8 t=8 3.01 -> 2.94, LL N=8 4.08 -> 4.04).
  auto after_sum = [&](int k) {
    if constexpr ((!NORM && !(STREAM && ALL_AT_ONCE)) || SPLIT) store_residual(k);
    if constexpr (NORM) {
      // h is fp32, so h * h is exact in fp64 and the fused multiply-add
      // rounds exactly as the separate product and sum would
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (ok[k][e / 4]) {
          const double hd = (double)h[k][e];
          ss = __builtin_fma(hd, hd, ss);
        }
    }
  };
  // refill this row of the slot set a later call reuses; done last, when the
  // row's data no longer occupy registers
  auto reset_row = [&]() {
    if constexpr (SENT) {
      if (a.flags & kReset) {
        if constexpr (!ALL_AT_ONCE) fresh_offsets();
        const u32x4 sv = {a.sentinel2, a.sentinel2, a.sentinel2, a.sentinel2};
#pragma unroll
        for (int k = 0; k < VPT; ++k)
          if (ok[k][0]) {
#pragma unroll
            for (int i = 0; i < N; ++i)
              store16(at_w<u32x4>((char*)a.reset[i] + rb * 2, eo[k][0] * 2), sv);
          }
      }
    }
  };

  // ---- the row's chunks
  if constexpr (ALL_AT_ONCE) {
    // every load of the row in flight before the first use; the scheduling
    // barrier keeps arithmetic out of the load block
#pragma unroll
    for (int k = 0; k < VPT; ++k) load_chunk(k);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < VPT; ++k) arrive(k);
    if constexpr (G_AFTER_ARRIVAL) {
#pragma unroll
      for (int k = 0; k < VPT; ++k) load_gamma(k);
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k) rank_sum(k);
    if constexpr (G_AFTER_SUM) {
#pragma unroll
      for (int k = 0; k < VPT; ++k) load_gamma(k);
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k) after_sum(k);
  } else {
    // wide rows: loads run D chunks ahead of the arithmetic (the barriers
    // stop the scheduler from hoisting every load to the top, which would
    // need more registers than a 1024-thread block has)
#pragma unroll
    for (int k = 0; k < D; ++k) load_chunk(k);
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      if (k > 0 && k + D - 1 < VPT) load_chunk(k + D - 1);
      __builtin_amdgcn_sched_barrier(0);
      arrive(k);
      rank_sum(k);
      after_sum(k);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  if (bad && a.status) {
    atomicAdd((unsigned long long*)&a.status->bad_words, (unsigned long long)bad);
    atomicOr(&a.status->code, (uint32_t)ARFUSE_ERR_FLAG_TIMEOUT);
  }
  if constexpr (!NORM) {
    // the all-reduce alone in a streaming row: residual_out after a
    // workgroup barrier, so the row's stores leave together once all of its
    // reads are in, as a normalizing row's do (t=4096: 111.5-111.7 ->
    // 110.7-110.9 us, without residual 96.8-97.4 -> 96.3-96.5)
    if constexpr (STREAM && ALL_AT_ONCE) {
      __syncthreads();
#pragma unroll
      for (int k = 0; k < VPT; ++k) store_residual(k);
    }
    reset_row();
    return;
  }

  // ---- row reduction: DPP tree inside each wave, one LDS slot per wave, then
  // every wave sums the (at most 16) slots with the same 16-lane tree
  __shared__ double red[kMaxBlock / kWave];
  ss = wave_sum<!SPLIT>(ss);
  if ((lane & (kWave - 1)) == 0) red[lane / kWave] = ss;
  __syncthreads();
  const int nw = nthr / kWave;
  const int wl = lane & (kWave - 1);
  double tot = lane_f64(row16_sum<!SPLIT>(wl < nw ? red[wl] : 0.0), 0);
  if constexpr (SPLIT) {
    // Split row: publish this slice's sum of squares tagged with this
    // dispatch's token, then lanes 0..split-1 of wave 0 wait (bounded) for
    // every partner slot to carry the same token; the partials are added in
    // slice order, so every slice computes the same total.
    // The slot is written twice, to two regions: into the L2 that the row's
    // slices share (they are placed on one XCD, above; store16_l2), and
    // through to memory (store16_through). Partners poll with the re-read
    // of the arrival checks (a volatile buffer load, which the compiler
    // issues with sc0 sc1; reread16_l2 is the same load): seven polls in
    // eight read the first copy, which
    // a partner on the same XCD finds in that XCD's L2, and every eighth
    // reads the second, so a placement that puts a partner on another XCD
    // costs time, never a result. Each row's slots fill one 128-byte line of
    // its own in each region, so the lines an XCD writes are written by no
    // other XCD. Against one region at slot b, written through, slices on
    // different XCDs: N = 8, t = 8, d = 8192 chains 3.20-3.30 -> 2.95 us (4
    // slices), LL 4.34-4.40 -> 4.09 us (8 slices), FP4 t = 1 3.04-3.19 ->
    // 2.86 us. Polls of the first copy with sc0 alone (not volatile, kept in
    // the loop by a compiler barrier) were 0.2-0.7 us slower per call.
    __shared__ double xsum;
    if (lane < kWave) {
      const u32x2 tok = dispatch_token();
      char* wsb = (char*)a.ws;
      const uint32_t region = prows * 128;  // bytes of one region
      const uint32_t wsbytes = 2 * region;
      if (lane == 0) {
        const uint64_t tb = (uint64_t)__double_as_longlong(tot);
        const u32x4 slot = {(uint32_t)tb, (uint32_t)(tb >> 32), tok.x, tok.y};
        const uint32_t own = (row * 8 + slice) * 16;
        store16_l2(wsb, wsbytes, own, slot);
        store16_through(wsb, wsbytes, region + own, slot);
      }
      double part = tot;
      uint32_t xbad = 0;
      if (lane < (1 << lg) && (uint32_t)lane != slice) {
        const uint32_t off = (row * 8 + (uint32_t)lane) * 16;
        u32x4 w = {0u, 0u, 0u, 0u};
        bool got = false;
        for (uint32_t i = 0; i < kExchangePolls; ++i) {
          w = (i & 7u) == 7u ? reread16(wsb, wsbytes, region + off) : reread16_l2(wsb, wsbytes, off);
          if ((w.z == tok.x) & (w.w == tok.y)) {
            got = true;
            break;
          }
          if (i >= 64) __builtin_amdgcn_s_sleep(1);
        }
        part = got ? __hiloint2double((int)w.y, (int)w.x) : 0.0;
        xbad = got ? 0u : 1u;
      }
      double sum = 0.0;
      for (int p = 0; p < (1 << lg); ++p) sum += lane_f64(part, p);
      if (lane == 0) xsum = sum;
      if (xbad && a.status) {
        atomicAdd(&a.status->exchange_timeouts, xbad);
        atomicOr(&a.status->code, (uint32_t)ARFUSE_ERR_FLAG_TIMEOUT);
      }
    }
    __syncthreads();
    tot = xsum;
  }
  // The row's scale in fp64, rounded once to fp32; each element is then
  // scaled with two fp32 multiplies, y = (h * inv) * gamma. In fp64 the
  // scaling took five instructions per element (two widenings, two
  // multiplies, a narrowing) in the part of the call that runs after the
  // row's loads have landed: 0.1-0.16 us of every decode call.
  const float inv = (float)inv_rms(tot, a.inv_d, (double)a.eps);

  // ---- normalize, scale by gamma, store bf16 / FP4 / FP8
  if constexpr (!ALL_AT_ONCE) {
    fresh_offsets();
    // keep h as floats: otherwise each (double)h of the sum of squares is
    // reused here, and a wide row's doubles need twice the registers
#pragma unroll
    for (int k = 0; k < VPT; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(h[k][e]));
    load_gamma(0);
  }
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    if constexpr (!ALL_AT_ONCE) {  // gamma one chunk ahead
      if (k + 1 < VPT) load_gamma(k + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    float y[8];
    const float gg[8] = {g[k][0].x, g[k][0].y, g[k][0].z, g[k][0].w,
                         g[k][1].x, g[k][1].y, g[k][1].z, g[k][1].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (h[k][e] * inv) * gg[e];
    if constexpr (!SPLIT) store_residual(k);
    if constexpr (OUT) {
      const u32x4 yb = narrow8(y);
      if constexpr (LL) {
        if (ok[k][0]) out_store<SPOL>(yrow, eo[k][0] * 2, u32x2{yb.x, yb.y});
        if (ok[k][1]) out_store<SPOL>(yrow, eo[k][1] * 2, u32x2{yb.z, yb.w});
      } else if (ok[k][0]) {
        out_store<SPOL>(yrow, eo[k][0] * 2, yb);
      }
    }
    if constexpr (FP8) {
      const uint32_t q[2] = {fp8_quad(y, a.fp8_inv_scale), fp8_quad(y + 4, a.fp8_inv_scale)};
      if constexpr (LL) {
        if (ok[k][0]) out_store<SPOL>(frow, eo[k][0], q[0]);
        if (ok[k][1]) out_store<SPOL>(frow, eo[k][1], q[1]);
      } else if (ok[k][0]) {
        out_store<SPOL>(frow, eo[k][0], u32x2{q[0], q[1]});
      }
    }
    if constexpr (FP4) {
      if constexpr (LL) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          uint32_t c4, sc;
          fp4_quad(y + 4 * j, c4, sc);
          if (ok[k][j]) {
            *at_w<uint16_t>(crow, eo[k][j] / 2) = (uint16_t)c4;
            if ((lane & 3) == 0) *at_w<uint8_t>(srow, eo[k][j] / 16) = (uint8_t)sc;
          }
        }
      } else {
        uint32_t c8, sc;
        fp4_pair(y, c8, sc);
        if (ok[k][0]) {
          out_store<SPOL>(crow, eo[k][0] / 2, c8);
          if ((eo[k][0] & 15) == 0) *at_w<uint8_t>(srow, eo[k][0] / 16) = (uint8_t)sc;
        }
      }
    }
  }
  reset_row();
}

typedef void (*RowFn)(RowArgs);

// Instances for one rank count: returns the kernel for (VPT, layout, EPI);
// layout is ARFUSE_LAYOUT_PLAIN, _LL or _SENTINEL.
RowFn select_row_kernel_n1(int vpt, int layout, int epi, int kind);
RowFn select_row_kernel_n2(int vpt, int layout, int epi, int kind);
RowFn select_row_kernel_n3(int vpt, int layout, int epi, int kind);
RowFn select_row_kernel_n4(int vpt, int layout, int epi, int kind);
RowFn select_row_kernel_n5(int vpt, int layout, int epi, int kind);
RowFn select_row_kernel_n6(int vpt, int layout, int epi, int kind);
RowFn select_row_kernel_n7(int vpt, int layout, int epi, int kind);
RowFn select_row_kernel_n8(int vpt, int layout, int epi, int kind);

}  // namespace arfuse_detail
